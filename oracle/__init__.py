"""fp64 CPU oracle of dynamic bifocal RoPE attention.  Test infrastructure:
only tests, the smoke check and the benchmark's CPU baseline use it."""
from .bifocal import (  # noqa: F401
    SKIP, LOCAL, REMOTE, STRADDLE, DIAG,
    group_size, remote_positions, rope_frequencies, rope_rotate,
    bifocal_sequence, bifocal_prefill, bifocal_rows, bifocal_decode,
    bifocal_sequence_ie, masked_attention, correction_rotation, tile_classes,
    bifocal_sequence_prerotated, bifocal_decode_prerotated,
)
