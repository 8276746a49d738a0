"""CPU oracle package.  TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline)."""
