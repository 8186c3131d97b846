"""CPU oracle for compressed-KV decode attention.  TEST INFRASTRUCTURE ONLY:
imported by the tests, the smoke check and the bench's CPU-baseline leg,
never by the product library."""
