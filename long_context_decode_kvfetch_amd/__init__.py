"""VerKV decode hot path (PoissonComp + KVFetch) for MI355X / gfx950."""
