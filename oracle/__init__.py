"""The oracle: a plain fp64 CPU statement of paged decode attention, the paged cache
write, the copy-on-write block clone and the block manager. Test infrastructure only."""
