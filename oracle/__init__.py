"""CPU oracle of the indexer: test infrastructure only (tests, smoke check,
benchmark CPU baseline).  The GPU path never imports this package."""
