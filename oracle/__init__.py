"""CPU reference of the sparse KV row resolver.  Test infrastructure only:
tests, the smoke check and the benchmark's CPU baseline use it; the product
path never does."""
