// tuning.hpp -- compile-time tuning constants of the HIP kernels.
#pragma once

// Compile-time tuning constants (defaults are the measured best on MI355X).
#ifndef SAGA_STREAM_U64
#define SAGA_STREAM_U64 2            // 16-row K groups per wave tile, head_dim 64
#endif
#ifndef SAGA_STREAM_U128
#define SAGA_STREAM_U128 1           // same, head_dim 128
#endif
#ifndef SAGA_K_NONTEMPORAL
#define SAGA_K_NONTEMPORAL 0         // stream K with non-temporal loads
#endif
#ifndef SAGA_TARGET_BLOCKS
#define SAGA_TARGET_BLOCKS 2048      // workgroups per stream launch (256 CUs)
#endif
