// tuning.hpp -- compile-time tuning constants of the HIP kernels.
#pragma once

// Compile-time tuning constants (defaults are the measured best on MI355X).
#ifndef SAGA_STREAM_U64
#define SAGA_STREAM_U64 1            // 16-row K groups per wave tile, head_dim 64
#endif
#ifndef SAGA_STREAM_U32
#define SAGA_STREAM_U32 1            // same, head_dim 32
#endif
#ifndef SAGA_STREAM_U128
#define SAGA_STREAM_U128 1           // same, head_dim 128
#endif
#ifndef SAGA_STREAM_K8_UMUL
#define SAGA_STREAM_K8_UMUL 1        // fp8 K: 16-row groups per tile, times the bf16 count
#endif
#ifndef SAGA_K_NONTEMPORAL
#define SAGA_K_NONTEMPORAL 0         // stream K with non-temporal loads
#endif
#ifndef SAGA_TARGET_BLOCKS64
#define SAGA_TARGET_BLOCKS64 768     // workgroups per K-stream launch, head_dim 64
#endif
#ifndef SAGA_TARGET_BLOCKS128
#define SAGA_TARGET_BLOCKS128 512    // same, head_dim 128
#endif
#ifndef SAGA_TARGET_BLOCKS32
#define SAGA_TARGET_BLOCKS32 1024    // same, head_dim 32 (64-byte rows, as fp8 at 64)
#endif
#ifndef SAGA_TARGET_BLOCKS64_K8
#define SAGA_TARGET_BLOCKS64_K8 1024 // same with an fp8 K cache, head_dim 64
#endif
#ifndef SAGA_TARGET_BLOCKS128_K8
#define SAGA_TARGET_BLOCKS128_K8 512 // same with an fp8 K cache, head_dim 128
#endif
#ifndef SAGA_GATHER_MAX_SEGS
#define SAGA_GATHER_MAX_SEGS 16      // most gather workgroups per (b, query head)
#endif
#ifndef SAGA_FULL_BLOCKS
#define SAGA_FULL_BLOCKS 512         // workgroups per dense (full-attention) launch
#endif
#ifndef SAGA_GATHER_NB
#define SAGA_GATHER_NB 4             // value rows in flight per lane in the gather
#endif
#ifndef SAGA_TAIL_GATHER
#define SAGA_TAIL_GATHER 1           // large-batch decode calls gather in the K stream's tail
#endif
#ifndef SAGA_TAIL_NB
#define SAGA_TAIL_NB 8               // value rows in flight per lane in that tail gather (d = 64)
#endif
#ifndef SAGA_TAIL_NB128
#define SAGA_TAIL_NB128 8            // same at d = 128
#endif
#ifndef SAGA_TAIL_NB_V8
#define SAGA_TAIL_NB_V8 3            // same with an fp8 V cache (16 codes per lane load)
#endif
#ifndef SAGA_GATHER_WAVES
#define SAGA_GATHER_WAVES 0          // >0: ask for that many waves per SIMD (gather)
#endif
#ifndef SAGA_STREAM_WAVES
#define SAGA_STREAM_WAVES 0          // >0: ask for that many waves per SIMD (K stream)
#endif
#if SAGA_GATHER_WAVES > 0
#define SAGA_GATHER_ATTR __attribute__((amdgpu_waves_per_eu(SAGA_GATHER_WAVES)))
#else
#define SAGA_GATHER_ATTR
#endif
#if SAGA_STREAM_WAVES > 0
#define SAGA_STREAM_ATTR __attribute__((amdgpu_waves_per_eu(SAGA_STREAM_WAVES)))
#else
#define SAGA_STREAM_ATTR
#endif
#ifndef SAGA_FUSED_MAX_GROUPS
#define SAGA_FUSED_MAX_GROUPS 4      // decode calls with at most this many (b, key head) groups
#endif                               // take the fused small-batch path
