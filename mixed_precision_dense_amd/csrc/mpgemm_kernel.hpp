// mpgemm_kernel.hpp -- the gfx950 MFMA GEMM kernel: D = alpha * op(A) * op(B) + beta * C.
//
// One workgroup of 4 waves (256 lanes, one wave per SIMD) computes a BM x BN tile of D.  The
// waves form a 2 x 2 grid; each owns a (BM/2) x (BN/2) sub-tile made of 16 x 16 MFMA blocks
// whose accumulators stay in the accumulation registers for the whole K loop.  K is walked in
// stages of 128 bytes per row (64 FP16/BF16 or 128 INT8 elements, two MFMA k steps of 64
// bytes).  Stages are copied from global memory straight into LDS by direct-to-LDS buffer
// loads (whole 128-byte lines per row) into free buffers -- two for A, three for B -- while
// the waves multiply out of another; each of a stage's two k steps queues half of the loads
// of the stage two ahead (B's in the first, A's in the second).
//
// The structure follows the pages' description of a tensor-core GEMM, re-planned for CDNA4:
//   * the product is a sum of rank-k slabs, each slab an outer product of a column panel of
//     A and a row panel of B ("The CUDA Handbook" section 17.5 "Tensor Cores", Figure 17-4);
//   * slabs are staged in on-chip shared memory in a block tile, each wave multiplying
//     fragments of it ("The CUDA Handbook" section 17.5, Listing 17-5 and the paragraph after
//     it, which also observes that the wait for the next slab's global load becomes the
//     bottleneck -- hence the stage buffers filled while another is multiplied here);
//   * the accumulator starts at zero, the K loop accumulates in place, and the epilogue scales
//     the product by alpha and adds beta * C element by element before storing
//     ("Programming Tensor Cores in CUDA 9", sections "Inner loop" and "Finishing");
//   * FP16/BF16 products are accumulated in FP32, INT8 products in INT32 ("Programming Tensor
//     Cores in CUDA 9", "What are Tensor Cores?"; "Mixed-Precision Programming with CUDA 8",
//     DP4A, Figure 2).
//
// Why 16 x 16 blocks: on random data the chip runs power-limited, and v_mfma_f32_16x16x32_*
// and v_mfma_i32_16x16x64_i8 do the same work as the 32 x 32 forms for 15-20 % less energy
// (measured: higher sustained clock at equal MFMA utilisation).  Their 16-cycle issue
// interval leaves room for two other instructions between MFMAs without delaying the next
// one, which is what the hand-placed schedule below is built around.
//
// MFMA lane layouts (probed on gfx950): every operand register set is 16 bytes per lane;
// lane l holds row (A) or column (B) l % 16 and the 16-byte k chunk l / 16 of the 64-byte k
// step.  Accumulator register r of lane l holds row 4 * (l / 16) + r, column l % 16.
//
// LDS layout: [A stage 0 | A stage 1 | B stage 0 | B stage 1 | B stage 2].  Each operand's
// stage is a row of 4 KB sub-tiles of 32 rows (K-contiguous) or a row of 128-byte column
// groups (MN-contiguous), so that fragment addresses differ only by immediate offsets.
//   * K-contiguous operand (A with transa = N, B with transb = T): sub-tile = 32 rows x 128 B,
//     16-byte chunk c of row r at chunk position c ^ kc_swz(r), which keeps a fragment read
//     free of bank conflicts (see kc_swz).
//   * MN-contiguous operand (A with transa = T, B with transb = N): the tile keeps its global
//     orientation, as k-rows of 128-byte column groups (four 16-column blocks for 16-bit
//     types, eight for 8-bit types), and is transposed on the way out of LDS by
//     ds_read_b64_tr_b16 / ds_read_b64_tr_b8.  Within a 16-lane group these return, to lane
//     t, element s of the row read by lane 4s + t/4 (b16) or 2s + t/8 (b8), at position t % 4
//     (t % 8) of that row.  Chunk c of k-row k sits at c ^ mn_swz(k).
//   One direct-to-LDS load of a wave fills 1 KB of LDS, lane l the 16 bytes at l * 16; the
//   lane-to-chunk mapping applies the swizzle on the global side.
//
// Edges are handled inside the same kernel (see the Operand comment): loads stay inside the
// operand through clamped offsets and an exact record count for the last stage, chunks past
// K are zeroed in LDS, and stores outside m x n are dropped through an out-of-range offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "mpgemm_kinds.hpp"

namespace mpg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) char lds_char;

// Kernel arguments (one struct, passed by value).
struct Params {
    const void *A;
    const void *B;
    const void *C;
    void *D;
    int64_t lda, ldb, ldc;  // elements
    int m, n, k;
    int tiles_m, tiles_n;
    float alpha_f, beta_f;
    int alpha_i, beta_i;
    int read_c;  // beta != 0
};

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, fully expanded in
// the source (the long MFMA sequences exceed what the unroller expands on request).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kStageKBytes = 128;   // bytes of k per row per stage (two MFMA k steps)
constexpr int kStepKBytes = 64;     // bytes of k per row per MFMA k step
constexpr int kSubTileBytes = 4096; // 32 rows x 128 B, or the transposed equivalent
constexpr int kBuffers = 2;         // LDS buffers of A's stages
// LDS buffers of B's stages: three, so that a stage's B loads can be queued a k step (FP8: a
// half stage) before its A loads (see gemm_tile)
constexpr int b_buffers(int) { return 3; }
constexpr int kGroupM = 4;          // tile-row grouping for L2 reuse
constexpr uint32_t kOobOffset = 0x80000000u;  // a buffer offset past every resource's range
constexpr int kNumRecords = 0x7FFFFFFF;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    // raw buffer, stride 0; dword3 selects 32-bit data format (required non-zero on gfx9)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, kNumRecords,
                                             0x00020000);
}

// An empty statement that uses a value held in scalar registers.  Placed where the value is
// computed (between two MFMAs), it keeps the compiler from sinking that scalar work past the
// k-tail branch into the block just before the next barrier, where the matrix cores would sit
// idle while it issues.
template <typename T>
__device__ __forceinline__ void keep_here(const T &v) {
    asm volatile("" : : "s"(v));
}

// The same raw-buffer descriptor as four dwords, for the direct-to-LDS load below.
__device__ __forceinline__ i32x4 make_rsrc_words(const void *base) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);   // stride 0, no swizzle
    r[2] = kNumRecords;
    r[3] = 0x00020000;
    return r;
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes [voff + soff, +16) of the buffer go
// to LDS address m0 + 16 l.  Written as inline assembly so that the compiler does not treat it
// as an LDS store: otherwise it would make every later transposed LDS read wait for all of
// these loads.  The kernel orders them itself: vmcnt waits before each barrier that publishes
// the data, and before any LDS access to it.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
}

// The same for C of a whole tile, whose every element is read once: non-temporal (the nt cache
// policy), so that C's stream leaves the L2 and the memory-side cache to the A and B panels that
// are read again.  D's whole-chunk stores from the LDS take the same policy (kStreamPolicy, the
// buffer builtins' cache-policy argument) -- when rows are whole 128-byte lines: non-temporal
// partial lines (unaligned row pitch, element-wise stores at tile edges) cost far more than the
// default policy, under which the L2 gathers them.
__device__ __forceinline__ void dma16_stream(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
}
constexpr int kStreamPolicy = 2;   // nt

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima): at most N of this wave's
// vector-memory loads are still in flight -- loads complete in order, so every older one has
// landed (for direct-to-LDS loads: its data is in LDS).  The compiler does not insert this
// wait for LDS-destination loads before a barrier by itself.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N & 0x30) << 10));
}

// s_waitcnt lgkmcnt(N) (vmcnt and expcnt left at their maxima): at most N of this wave's LDS
// (and scalar memory) operations are still outstanding.
template <int N>
__device__ __forceinline__ void wait_lds() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// Zero the bytes of a 16-byte chunk at and beyond byte `nbytes` (0..16).
__device__ __forceinline__ u32x4 keep_first_bytes(u32x4 v, int nbytes) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int left = nbytes - 4 * j;
        const uint32_t mask = left >= 4 ? 0xFFFFFFFFu : (left <= 0 ? 0u : ((1u << (8 * left)) - 1u));
        v[j] &= mask;
    }
    return v;
}

// ---------------------------------------------------------------------------------------
// Operand stage: global -> LDS copy and LDS -> MFMA fragment reads.
//   EB: element bytes (2 or 1).  KC: K-contiguous storage.  NS: number of 32-row (A) or
//   32-column (B) sub-tiles in the tile, i.e. 2 NS fragment blocks of 16.
//
// Loads never leave the operand.  K-contiguous rows outside the tile's m (or n) range are
// clamped to the last valid row and MN-contiguous chunks past the row end to its last
// 16-byte block, so every stage but the last stays inside rows that exist.  For the last stage the buffer resource's record
// count is the exact number of guaranteed-readable bytes from the stage start (and zero for
// stages past K), so chunks beyond the operand's end read as zero.  Data loaded for rows or
// columns outside m x n only reaches accumulators of outputs that are never stored.  Chunks
// beyond K within a row are the exception -- they would reach every output -- and are zeroed
// in LDS once they have landed (fix_k_tail).
// ---------------------------------------------------------------------------------------
template <int EB, bool KC, int NS, int R = 1>
struct Operand {
    static_assert(NS == 2 || NS == 4 || NS == 8, "sub-tile count");
    static_assert((R == 1 || R == 2) && NS % R == 0, "waves per quarter slot");
    static constexpr int kStageBytes = NS * kSubTileBytes;
    static constexpr int kChunkElems = 16 / EB;             // elements per 16-byte chunk
    static constexpr int kSlots = NS / R;                   // 1 KB loads per wave per stage
    static constexpr int kStageK = kStageKBytes / EB;       // k elements per stage
    static constexpr int kStepK = kStepKBytes / EB;         // k elements per MFMA k step
    // MN-contiguous geometry: k-rows of 128-byte column groups, kGroupBlocks 16-wide fragment
    // blocks each (4 for 16-bit, 8 for 8-bit types), so that every direct load moves whole
    // 128-byte lines.
    static constexpr int kGroupBlocks = 128 / (16 * EB);
    static constexpr int kGroupBytes = kStageK * 128;       // one column group of a stage
    static constexpr int kSlotsPerGroup = kStageK / 32;     // 2 (16-bit) or 4 (8-bit)
    static_assert(KC || 2 * NS >= kGroupBlocks, "transposed operand needs whole column groups");

    // The stage is cut into 1 KB quarters, four per 4 KB sub-tile position o (0 .. NS - 1);
    // quarter v of position o sits at o * 4096 + v * 1024, lane l's 16 bytes at l * 16: for a
    // K-contiguous operand quarter v of sub-tile o (8 rows x 128 B), for an MN-contiguous one
    // rows 32 (o % kSlotsPerGroup) + 8 v .. + 7 of column group o / kSlotsPerGroup.  With 4R
    // waves, wave w loads quarter v = w % 4 of the positions o = i R + w / 4, its slots
    // i = 0 .. kSlots - 1.
    uint32_t voff[kSlots];  // per slot: byte offset of this lane's chunk from the stage start
    // fragment read offsets: K-contig per k step; MN-contig per block position in its group
    uint32_t r_off[kGroupBlocks > 2 ? kGroupBlocks : 2];

    // Chunk swizzle of a K-contiguous row r of a sub-tile (chunk c sits at c ^ kc_swz(r)):
    // bits 1 and 2 of (r mod 16) / 2 swapped.  A fragment read (16 rows x 64 bytes) is served
    // by the LDS 32 lanes at a time over 128 four-byte banks (measured on gfx950: lanes 0-31,
    // then 32-63); lanes 0-31 read rows 0..15 at two adjacent chunks, and rows r, r + 4, r + 8,
    // r + 12 share a bank base, so their swizzles must fall in distinct pairs {c, c ^ 1}.
    static __device__ __forceinline__ int kc_swz(int r) {
        const int j = (r & 15) >> 1;
        return (j & 1) | ((j & 2) << 1) | ((j & 4) >> 1);
    }
    // Chunk swizzle of an MN-contiguous k-row (chunk c of row k sits at c ^ mn_swz(k)).
    static __device__ __forceinline__ int mn_swz(int k) {
        return EB == 2 ? 2 * ((k & 3) ^ ((k >> 3) & 1)) : ((k & 7) ^ ((k >> 4) & 1));
    }

    // mn_left: rows (K-contig) or columns (MN-contig) of the operand from the tile's first
    // one; at least 1.
    // lds_base: byte offset of this operand's stages in LDS, folded into the read offsets.
    // wave: the quarter v this wave loads (wave index mod 4); hi: the wave index / 4.
    __device__ __forceinline__ void init(int wave, int hi, int lane, int64_t ld, int mn_left,
                                         uint32_t lds_base) {
        const uint32_t row_bytes = (uint32_t)(ld * EB);
        const int g = lane / 16, u = lane % 16;
        if constexpr (KC) {
            const int r = wave * 8 + lane / 8;                      // row within the sub-tile
            const int c = (lane % 8) ^ kc_swz(r);                   // logical chunk of phys lane % 8
#pragma unroll
            for (int i = 0; i < kSlots; ++i)
                voff[i] = (uint32_t)min(32 * (i * R + hi) + r, mn_left - 1) * row_bytes + 16u * c;
            // fragment: lane reads row u of its 16-row block, chunk g of the 64-byte k step
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                r_off[ks] = lds_base + (uint32_t)(u * 128 + 16 * ((4 * ks + g) ^ kc_swz(u)));
        } else {
            const int kr = wave * 8 + lane / 8;                     // k-row within a 32-row slot
            const int c = (lane % 8) ^ mn_swz(kr);                  // logical chunk in the group
            // chunks past the operand's row end (edge tiles) are clamped to its last 16-byte
            // block, so no load runs into later rows
            const int col_max = ((mn_left * EB + 15) & ~15) - 16;
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                const int o = i * R + hi;                           // sub-tile position
                voff[i] = (uint32_t)(32 * (o % kSlotsPerGroup) + kr) * row_bytes +
                          (uint32_t)min((o / kSlotsPerGroup) * 128 + 16 * c, col_max);
            }
            if constexpr (EB == 2) {
                // tr16: lane 4 s + q of group g reads k-row 8 g + s (+4 for the high half),
                // 8 bytes at column 4 q of its 16-column block
                const int s = u >> 2, q = u & 3, k = 8 * g + s;
#pragma unroll
                for (int pb = 0; pb < kGroupBlocks; ++pb)
                    r_off[pb] = lds_base + (uint32_t)(k * 128 + 16 * ((2 * pb + (q >> 1)) ^ mn_swz(k)) + 8 * (q & 1));
            } else {
                // tr8: lane 2 s + q of group g reads k-row 16 g + s (+8 for the high half),
                // 8 bytes at column 8 q of its 16-column block
                const int s = u >> 1, q = u & 1, k = 16 * g + s;
#pragma unroll
                for (int pb = 0; pb < kGroupBlocks; ++pb)
                    r_off[pb] = lds_base + (uint32_t)(k * 128 + 16 * (pb ^ mn_swz(k)) + 8 * q);
            }
        }
    }

    // Queue load slot i of a stage: rs addresses the stage's start (record count bounded as
    // described above), lds_stage_w is the LDS address of the stage plus this wave's
    // 4096 * hi + 1024 * wave.
    __device__ __forceinline__ void load(i32x4 rs, uint32_t lds_stage_w, int i) const {
        dma16(rs, voff[i], 0u, lds_stage_w + (uint32_t)(i * R) * 4096u);
    }

    // After the last stage has landed, when K ends inside it: zero this lane's K-contiguous
    // chunks at and past K (whole chunks past K, the tail of the chunk that straddles it).
    // MN-contiguous k-rows past K lie beyond the operand and were read as zeros.  The lane's
    // chunk position is recomputed here (from an opaque copy of the lane index), so that none
    // of it is held in registers across the K loop.
    __device__ __forceinline__ void fix_k_tail(lds_char *stage, int k_left, int wave, int hi,
                                               int lane) const {
        if constexpr (KC) {
            asm volatile("" : "+v"(lane));
            const int r = wave * 8 + lane / 8;
            const int k0 = ((lane % 8) ^ kc_swz(r)) * kChunkElems;   // first k of its chunks
            const uint32_t l_off = (uint32_t)(hi * 4096 + wave * 1024 + lane * 16);
            const int kvalid = k_left - k0;
            if (kvalid < kChunkElems) {
                const int keep = kvalid > 0 ? kvalid * EB : 0;
#pragma unroll
                for (int i = 0; i < kSlots; ++i) {
                    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
                    lds_u32x4 *q = (lds_u32x4 *)(stage + i * R * 4096 + l_off);
                    *q = keep_first_bytes(*q, keep);
                }
            }
        }
    }

    // Fragment reads as a base register plus an immediate: kReadBases bases per stage buffer
    // and wave (K-contiguous: one per k step; MN-contiguous: one per block position in a column
    // group), each read_base(stage LDS address, i, the wave's first block), which for an
    // MN-contiguous operand must be a multiple of kGroupBlocks.
    static constexpr int kReadBases = KC ? 2 : kGroupBlocks;
    __device__ __forceinline__ uint32_t read_base(uint32_t stage_addr, int i, int first_blk) const {
        if constexpr (KC)
            return stage_addr + r_off[i] + (uint32_t)(first_blk * 16 * kStageKBytes);
        else
            return stage_addr + r_off[i] + (uint32_t)((first_blk / kGroupBlocks) * kGroupBytes);
    }
    // Fragment of the wave's block j at k step ks from its base: base index ks (K-contiguous)
    // or j mod kGroupBlocks (MN-contiguous).
    __device__ __forceinline__ u32x4 frag_at(uint32_t base, int j, int ks) const {
        typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
        if constexpr (KC) {
            return *(const lds_u32x4 *)(lds_char *)(uintptr_t)(base + (uint32_t)(j * 16 * kStageKBytes));
        } else if constexpr (EB == 2) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const uint32_t a = base + (uint32_t)((j / kGroupBlocks) * kGroupBytes + ks * kStepK * 128);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lds_char *)(uintptr_t)a);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lds_char *)(uintptr_t)(a + 4 * 128));
            return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
            const uint32_t a = base + (uint32_t)((j / kGroupBlocks) * kGroupBytes + ks * kStepK * 128);
            const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(lds_char *)(uintptr_t)a);
            const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(lds_char *)(uintptr_t)(a + 8 * 128));
            return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
        }
    }

    // 16-byte MFMA operand of 16-wide block `blk` at k step `ks` (0 or 1) of a stage; `stage`
    // is the LDS start plus the stage's offset from this operand's first stage.
    __device__ __forceinline__ u32x4 frag(const lds_char *stage, int blk, int ks) const {
        if constexpr (KC) {
            return *(const __attribute__((address_space(3))) u32x4 *)(stage + blk * 2048 + r_off[ks]);
        } else if constexpr (EB == 2) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const lds_char *p = stage + (blk / kGroupBlocks) * kGroupBytes + r_off[blk % kGroupBlocks] + ks * kStepK * 128;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * 128));
            // register concatenation only: no arithmetic waits on the reads here
            return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
            const lds_char *p = stage + (blk / kGroupBlocks) * kGroupBytes + r_off[blk % kGroupBlocks] + ks * kStepK * 128;
            const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p));
            const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p + 8 * 128));
            return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
        }
    }
};

// Buffer resource of one operand's stages: the address of the next stage to load and the
// record count of the last stage (the exact number of guaranteed-readable bytes from its
// start, computed once per tile).
struct StageCursor {
    uint64_t base;      // global address of the next stage's start
    int64_t step;       // bytes between consecutive stages
    int last_records;   // record count for the last stage
    __device__ __forceinline__ void advance() { base += (uint64_t)step; }
    // Resource for stage s of nk: every byte before the last stage, exact for the last
    // stage, none past it.
    __device__ __forceinline__ i32x4 rsrc(int s, int nk) const {
        return words(s < nk - 1 ? kNumRecords : (s == nk - 1 ? last_records : 0));
    }
    // The resource of the next stage with record count nr.
    __device__ __forceinline__ i32x4 words(int nr) const {
        i32x4 r;
        r[0] = (int)(uint32_t)base;
        r[1] = (int)((uint32_t)(base >> 32) & 0xFFFFu);   // stride 0, no swizzle
        r[2] = nr;
        r[3] = 0x00020000;
        return r;
    }
};

// ---------------------------------------------------------------------------------------
// MFMA per input type: one 16 x 16 block, 64 bytes of k per row (32 FP16/BF16 or 64 INT8).
// The accumulators are pinned to the accumulation registers through the asm operand
// constraint; every other register holds fragments, offsets and the loop state.  An
// accumulator is next used as an input 64 (or, for smaller tiles, 16 or 4) MFMAs later, and
// the epilogue waits out the last results (drain_mfma) before reading them.
// ---------------------------------------------------------------------------------------
template <int IN> struct Mma;
template <> struct Mma<IN_F16> {
    typedef f32x4 acc_t;
    static __device__ __forceinline__ void run(u32x4 a, u32x4 b, acc_t &c) {
        asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct Mma<IN_BF16> {
    typedef f32x4 acc_t;
    static __device__ __forceinline__ void run(u32x4 a, u32x4 b, acc_t &c) {
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct Mma<IN_I8> {
    typedef i32x4 acc_t;
    static __device__ __forceinline__ void run(u32x4 a, u32x4 b, acc_t &c) {
        asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};
// FP8: one 16 x 16 block over a whole 128-byte stage (128 k).  Operand registers: the two
// 16-byte fragments of the stage's k steps (low half k step 0, high half k step 1), the same
// for A and B, so both operands present their k in the same order.  cbsz / blgp select the
// A / B formats (0 = E4M3, 1 = E5M2).
template <int IN> struct Mma8;
template <> struct Mma8<IN_FP8_FP8> {
    static __device__ __forceinline__ void run(u32x8 a, u32x8 b, f32x4 &c) {
        asm("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:0 blgp:0" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct Mma8<IN_FP8_BF8> {
    static __device__ __forceinline__ void run(u32x8 a, u32x8 b, f32x4 &c) {
        asm("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:0 blgp:1" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct Mma8<IN_BF8_FP8> {
    static __device__ __forceinline__ void run(u32x8 a, u32x8 b, f32x4 &c) {
        asm("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:0" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct Mma8<IN_BF8_BF8> {
    static __device__ __forceinline__ void run(u32x8 a, u32x8 b, f32x4 &c) {
        asm("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <int IN> struct MmaAcc { typedef typename Mma<IN>::acc_t type; };
template <> struct MmaAcc<IN_FP8_FP8> { typedef f32x4 type; };
template <> struct MmaAcc<IN_FP8_BF8> { typedef f32x4 type; };
template <> struct MmaAcc<IN_BF8_FP8> { typedef f32x4 type; };
template <> struct MmaAcc<IN_BF8_BF8> { typedef f32x4 type; };

// Half h (0 or 1) of an 8-dword fragment register (element inserts: the compiler writes the
// loaded registers in place, without copies).
__device__ __forceinline__ void set_half(u32x8 &v, int h, u32x4 x) {
    if (h == 0) {
        v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
    } else {
        v[4] = x[0]; v[5] = x[1]; v[6] = x[2]; v[7] = x[3];
    }
}

// Wait states between the last MFMA of the loop and the first read of its results by any
// other instruction (more than an 8-pass MFMA's result latency), then every accumulator is
// passed through an empty volatile statement, so no read of it can be scheduled earlier.
template <typename Acc, int FM, int FN>
__device__ __forceinline__ void drain_mfma(Acc (&acc)[FM][FN]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// ---------------------------------------------------------------------------------------
// Epilogue element: v = fma(alpha, acc, beta * c) in FP32 (v = alpha * acc when beta == 0, and C
// is not read), converted to the output type with one round-to-nearest-even.
// ---------------------------------------------------------------------------------------
template <int OUT> struct Out;
template <> struct Out<OUT_F32> {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ float lds_load(const lds_char *q) {
        return *(const __attribute__((address_space(3))) float *)q;
    }
    static __device__ __forceinline__ void lds_store(lds_char *q, float v) {
        *(__attribute__((address_space(3))) float *)q = v;
    }
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
    }
};
template <> struct Out<OUT_F16> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float lds_load(const lds_char *q) {
        return (float)*(const __attribute__((address_space(3))) _Float16 *)q;
    }
    static __device__ __forceinline__ void lds_store(lds_char *q, float v) {
        asm("" : "+v"(v));   // the FP32 value, then one RNE conversion (see store)
        *(__attribute__((address_space(3))) _Float16 *)q = (_Float16)v;
    }
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
        // The FP32 value first, then v_cvt_f16_f32 (round to nearest even under the default
        // mode).  The empty asm keeps the compiler from folding the epilogue's fma and this
        // conversion into v_fma_mixlo_f16, which rounds the exact result once, to FP16.
        asm("" : "+v"(v));
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (_Float16)v), r, (int)off, 0, 0);
    }
};
template <> struct Out<OUT_BF16> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float lds_load(const lds_char *q) {
        const uint32_t h = *(const __attribute__((address_space(3))) unsigned short *)q;
        return __builtin_bit_cast(float, h << 16);
    }
    static __device__ __forceinline__ void lds_store(lds_char *q, float v) {
        *(__attribute__((address_space(3))) unsigned short *)q =
            __builtin_bit_cast(unsigned short, (__bf16)v);
    }
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
        return __builtin_bit_cast(float, h << 16);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
        // gfx950 converts FP32 -> BF16 with round to nearest even
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, (int)off, 0, 0);
    }
};
template <> struct Out<OUT_I32> {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ int lds_load(const lds_char *q) {
        return *(const __attribute__((address_space(3))) int *)q;
    }
    static __device__ __forceinline__ void lds_store(lds_char *q, int v) {
        *(__attribute__((address_space(3))) int *)q = v;
    }
    static __device__ __forceinline__ int load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, int v) {
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, r, (int)off, 0, 0);
    }
};

// Map a workgroup id to its (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the 8 XCDs, 32 per XCD and round of 256 tiles.  Each XCD's tiles of a round form a block of
// 4 tile rows by 8 tile columns, so that they share A row panels and B column panels in that
// XCD's L2 (4 + 8 panels, the least 32 whole tiles can take).  When both tile counts are
// multiples of 16, a round's 256 tiles form a 16 x 16 region (the eight XCDs' blocks side by
// side: 16 A and 16 B panels from beyond the L2s per round instead of 32 and 8), and the
// regions follow each other in a serpentine, so that consecutive rounds share their A or B
// panels in the memory-side cache.  Otherwise ids are remapped so that each XCD receives a
// contiguous run of tiles, laid out in groups of kGroupM tile rows.
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int &tm, int &tn) {
    if (tiles_m % 16 == 0 && tiles_n % 16 == 0) {
        const int xcd = wg % 8, j = wg / 8, round = j / 32, i = j % 32;
        const int regions_n = tiles_n / 16;
        const int ra = round / regions_n, rb0 = round % regions_n;
        const int rb = (ra & 1) ? regions_n - 1 - rb0 : rb0;
        tm = 16 * ra + 4 * (xcd % 4) + i % 4;
        tn = 16 * rb + 8 * (xcd / 4) + i / 4;
        return;
    }
    const int total = tiles_m * tiles_n;
    const int per_xcd = total / 8;
    int id = wg;
    if (wg < per_xcd * 8) id = (wg % 8) * per_xcd + wg / 8;
    const int group_tiles = kGroupM * tiles_n;
    const int group = id / group_tiles;
    const int first_m = group * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int in_group = id - group * group_tiles;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// ---------------------------------------------------------------------------------------
// Epilogue of one tile: D = alpha * acc + beta * C, masked to m x n.  kInt: INT32 wrap-around
// arithmetic (INT8 inputs), else FP32 (see Out<>).  The 2 x (NW / 2) waves each hold FM x FN
// 16 x 16 blocks of a BM x BN tile.
// ---------------------------------------------------------------------------------------
template <bool kInt, int OUT, int FM, int FN, int BM, int BN, bool kFull, int NW = 4,
          typename AccT>
__device__ __forceinline__ void store_tile(const Params &p, AccT (&acc)[FM][FN], int m0, int n0,
                                           int wm, int wn, int lane, int m_left, int n_left) {
    constexpr int OB = Out<OUT>::kBytes;
    const int64_t tile_off = ((int64_t)m0 * p.ldc + n0) * OB;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char *)p.D + tile_off);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const char *)(p.read_c ? p.C : p.D) + tile_off);
    const uint32_t ldc_b = (uint32_t)(p.ldc * OB);
    // accumulator register r of block (i, j): row 16 i + 4 (lane / 16) + r, column 16 j + lane % 16
    const int row_base = wm * (BM / 2) + 4 * (lane / 16);
    const int col_base = wn * (BN / (NW / 2)) + (lane % 16);
    // byte offset of accumulator element r of block (i, j), or an out-of-range offset
    auto out_off = [&](int i, int j, int r) -> uint32_t {
        const int row = row_base + i * 16 + r;
        const int col = col_base + j * 16;
        const uint32_t off = (uint32_t)row * ldc_b + (uint32_t)col * OB;
        if constexpr (kFull) return off;
        return ((row < m_left) & (col < n_left)) ? off : kOobOffset;
    };
    if (p.read_c) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                decltype(Out<OUT>::load(rc, 0)) cv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) cv[r] = Out<OUT>::load(rc, out_off(i, j, r));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (kInt) {
                        const uint32_t v = (uint32_t)p.alpha_i * (uint32_t)acc[i][j][r] +
                                           (uint32_t)p.beta_i * (uint32_t)cv[r];
                        Out<OUT>::store(rd, out_off(i, j, r), (int)v);
                    } else {
                        // one rounding of beta * c, then alpha * acc + (beta * c) fused
                        Out<OUT>::store(rd, out_off(i, j, r),
                                        __builtin_fmaf(p.alpha_f, acc[i][j][r], p.beta_f * cv[r]));
                    }
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (kInt)
                        Out<OUT>::store(rd, out_off(i, j, r), (int)((uint32_t)p.alpha_i * (uint32_t)acc[i][j][r]));
                    else
                        Out<OUT>::store(rd, out_off(i, j, r), p.alpha_f * acc[i][j][r]);
                }
    }
}

// ---------------------------------------------------------------------------------------
// Epilogue of one tile when C is read (beta != 0): the arithmetic of store_tile, with C
// streamed through the LDS (free once the K loop is over: the caller has passed a barrier
// after every wave's last loads and fragment reads) so that its loads are issued well ahead
// of their use instead of block by block.  Each wave owns a quarter of the LDS as kSlots
// slots of one block row (16 rows of its sub-tile): direct-to-LDS loads of whole 16-byte
// chunks fill the slots ahead, and a slot is refilled with the block row kSlots further on as
// soon as its values have been read.  Vector-memory operations of a wave complete in order,
// so the wait for a block row counts the loads and stores issued after it.  Within a slot
// the chunks of row rho sit at chunk position c ^ swz(rho), so that the four rows one
// accumulator read touches fall on different LDS banks.  Chunks outside m x n are not read
// (out-of-range offsets give zeros) and the elements they would feed are not stored.
// ---------------------------------------------------------------------------------------
// Number of vector-memory operations issued after the C loads of block row i, up to its wait:
// loads of block rows 0 .. S-1 first, then per block row t its St stores followed by the loads
// of block row t + S (L per block row).
constexpr int c_ops_after(int i, int S, int FM, int L, int St) {
    int pos = 0, done_i = -1;
    for (int t = 0; t < S && t < FM; ++t) {
        pos += L;
        if (t == i) done_i = pos;
    }
    for (int t = 0; t < FM; ++t) {
        if (t == i) return pos - done_i;
        pos += St;
        if (t + S < FM) {
            pos += L;
            if (t + S == i) done_i = pos;
        }
    }
    return 0;
}

template <bool kInt, int OUT, int FM, int FN, int BM, int BN, int kRegionBytes, bool kFull,
          int NW, typename AccT>
__device__ __forceinline__ void store_tile_c_staged(const Params &p, AccT (&acc)[FM][FN], int m0,
                                                    int n0, int wm, int wn, int lane, int m_left,
                                                    int n_left, const lds_char *region,
                                                    uint32_t region_addr) {
    constexpr int OB = Out<OUT>::kBytes;
    constexpr int WR = BM / 2, WC = BN / (NW / 2);          // the wave's sub-tile
    constexpr int RB = WC * OB;                             // bytes of one sub-tile row
    constexpr int kCPR = RB / 16;                           // 16-byte chunks per row
    constexpr int kSlotBytes = 16 * RB;                     // one block row
    constexpr int L = kSlotBytes / 1024;                    // 1 KB direct loads per block row
    constexpr int S = kRegionBytes / kSlotBytes < FM ? kRegionBytes / kSlotBytes : FM;
    constexpr int St = FN * 4;                              // stores per block row
    static_assert(RB >= 16 && kSlotBytes % 1024 == 0 && S >= 1, "C staging geometry");
    static_assert(WR == 16 * FM && WC == 16 * FN, "sub-tile shape");
    using CT = decltype(Out<OUT>::lds_load(nullptr));   // float, or int for INT32 C

    const int64_t tile_off = ((int64_t)m0 * p.ldc + n0) * OB;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char *)p.D + tile_off);
    const i32x4 rc_words = make_rsrc_words((const char *)p.C + tile_off);
    const uint32_t ldc_b = (uint32_t)(p.ldc * OB);
    const int row0 = wm * WR, col0 = wn * WC;               // sub-tile origin within the tile
    auto swz = [](int rho) { return (((rho & 15) >> 2) * OB) & (kCPR - 1); };

    // Lane l of load q of a block row fills slot bytes q KB + 16 l: row rho, physical chunk
    // cp, which holds logical chunk cp ^ swz(rho).
    auto load_block_row = [&](int i, int slot) {
#pragma unroll
        for (int q = 0; q < L; ++q) {
            const int pos = q * 1024 + 16 * lane;
            const int rho = pos / RB;
            const int c = ((pos % RB) / 16) ^ swz(rho);
            const int row = row0 + 16 * i + rho;
            const int col = col0 + c * (16 / OB);
            uint32_t voff = (uint32_t)row * ldc_b + (uint32_t)col * OB;
            if constexpr (!kFull) voff = ((row < m_left) & (col < n_left)) ? voff : kOobOffset;
            dma16(rc_words, voff, 0u, region_addr + (uint32_t)(slot * kSlotBytes + q * 1024));
        }
    };
    // accumulator register r of block (i, j): row 16 i + 4 (lane / 16) + r, column 16 j + lane % 16
    const int g = lane / 16, u = lane % 16;
    const int row_base = row0 + 4 * g;
    const int col_base = col0 + u;
    auto out_off = [&](int i, int j, int r) -> uint32_t {
        const int row = row_base + i * 16 + r;
        const int col = col_base + j * 16;
        const uint32_t off = (uint32_t)row * ldc_b + (uint32_t)col * OB;
        if constexpr (kFull) return off;
        return ((row < m_left) & (col < n_left)) ? off : kOobOffset;
    };
    // byte offset within a slot of this lane's element of row 4 g + r, block column j
    auto c_at = [&](int j, int r) -> int {
        const int colb = (16 * j + u) * OB;                 // byte column in the row
        return (4 * g + r) * RB + ((((colb >> 4) ^ swz(4 * g + r))) << 4) + (colb & 15);
    };

    static_for<S>([&](auto t_c) { load_block_row(decltype(t_c)::value, decltype(t_c)::value); });
    static_for<FM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int after = c_ops_after(i, S, FM, L, St);
        wait_vmem<(after < 63 ? after : 63)>();          // block row i's C is in its slot
        const lds_char *slot = region + (i % S) * kSlotBytes;
        CT cv[FN][4];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) cv[j][r] = Out<OUT>::lds_load(slot + c_at(j, r));
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (kInt) {
                    const uint32_t v = (uint32_t)p.alpha_i * (uint32_t)acc[i][j][r] +
                                       (uint32_t)p.beta_i * (uint32_t)cv[j][r];
                    Out<OUT>::store(rd, out_off(i, j, r), (int)v);
                } else {
                    // one rounding of beta * c, then alpha * acc + (beta * c) fused
                    Out<OUT>::store(rd, out_off(i, j, r),
                                    __builtin_fmaf(p.alpha_f, acc[i][j][r], p.beta_f * cv[j][r]));
                }
            }
        if constexpr (i + S < FM) {
            wait_lds<0>();                                  // the slot's values are in registers
            load_block_row(i + S, i % S);
        }
    });
}

// ---------------------------------------------------------------------------------------
// Epilogue of a whole tile (no edge) through the LDS: the same arithmetic as store_tile (and,
// with kReadC, C streamed through the slots as in store_tile_c_staged), but each wave writes
// its block row of results into its slot in the row-major, chunk-swizzled layout and stores
// it to D by whole 16-byte chunks, row by row (a 1 KB store instruction covers two to eight
// full rows of the sub-tile instead of four 64- or 32-byte pieces of sixteen rows).  The
// caller has passed a barrier after every wave's last loads and fragment reads.
// ---------------------------------------------------------------------------------------
template <bool kInt, int OUT, int FM, int FN, int BM, int BN, int kRegionBytes, int NW,
          bool kReadC, bool kNT, typename AccT>
__device__ __forceinline__ void store_full_tile_staged(const Params &p, AccT (&acc)[FM][FN],
                                                       int m0, int n0, int wm, int wn, int lane,
                                                       lds_char *region, uint32_t region_addr) {
    constexpr int OB = Out<OUT>::kBytes;
    constexpr int WR = BM / 2, WC = BN / (NW / 2);          // the wave's sub-tile
    constexpr int RB = WC * OB;                             // bytes of one sub-tile row
    constexpr int kCPR = RB / 16;                           // 16-byte chunks per row
    constexpr int kSlotBytes = 16 * RB;                     // one block row
    constexpr int L = kSlotBytes / 1024;                    // 1 KB loads (stores) per block row
    constexpr int S = kRegionBytes / kSlotBytes < FM ? kRegionBytes / kSlotBytes : FM;
    static_assert(RB >= 16 && kSlotBytes % 1024 == 0 && S >= 1, "staging geometry");
    static_assert(WR == 16 * FM && WC == 16 * FN, "sub-tile shape");
    using CT = decltype(Out<OUT>::lds_load(nullptr));   // float, or int for INT32 C

    const int64_t tile_off = ((int64_t)m0 * p.ldc + n0) * OB;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char *)p.D + tile_off);
    const i32x4 rc_words = make_rsrc_words((const char *)(kReadC ? p.C : p.D) + tile_off);
    const uint32_t ldc_b = (uint32_t)(p.ldc * OB);
    const int row0 = wm * WR, col0 = wn * WC;               // sub-tile origin within the tile
    auto swz = [](int rho) { return (((rho & 15) >> 2) * OB) & (kCPR - 1); };
    // Byte offset in D (from the tile's origin) of the chunk at slot bytes q KB + 16 lane of
    // block row i: row rho, physical chunk cp, holding logical chunk cp ^ swz(rho).
    auto chunk_off = [&](int i, int q) -> uint32_t {
        const int pos = q * 1024 + 16 * lane;
        const int rho = pos / RB;
        const int c = ((pos % RB) / 16) ^ swz(rho);
        return (uint32_t)(row0 + 16 * i + rho) * ldc_b + (uint32_t)(col0 + c * (16 / OB)) * OB;
    };
    auto load_block_row = [&](int i, int slot) {
#pragma unroll
        for (int q = 0; q < L; ++q)
            (kNT ? dma16_stream : dma16)(rc_words, chunk_off(i, q), 0u,
                  region_addr + (uint32_t)(slot * kSlotBytes + q * 1024));
    };
    // byte offset within a slot of this lane's accumulator element of row 4 g + r, block
    // column j (accumulator register r of block (i, j) is row 16 i + 4 (lane / 16) + r,
    // column 16 j + lane % 16)
    const int g = lane / 16, u = lane % 16;
    auto c_at = [&](int j, int r) -> int {
        const int colb = (16 * j + u) * OB;                 // byte column in the row
        return (4 * g + r) * RB + ((((colb >> 4) ^ swz(4 * g + r))) << 4) + (colb & 15);
    };

    if constexpr (kReadC)
        static_for<S>([&](auto t_c) { load_block_row(decltype(t_c)::value, decltype(t_c)::value); });
    static_for<FM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        lds_char *slot = region + (i % S) * kSlotBytes;
        CT cv[FN][4];
        if constexpr (kReadC) {
            constexpr int after = c_ops_after(i, S, FM, L, L);
            wait_vmem<(after < 63 ? after : 63)>();      // block row i's C is in its slot
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) cv[j][r] = Out<OUT>::lds_load(slot + c_at(j, r));
        } else if constexpr (i >= S) {
            wait_lds<0>();       // the slot's previous block row has been read back
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (kInt) {
                    uint32_t v = (uint32_t)p.alpha_i * (uint32_t)acc[i][j][r];
                    if constexpr (kReadC) v += (uint32_t)p.beta_i * (uint32_t)cv[j][r];
                    Out<OUT>::lds_store(slot + c_at(j, r), (int)v);
                } else if constexpr (kReadC) {
                    // one rounding of beta * c, then alpha * acc + (beta * c) fused
                    Out<OUT>::lds_store(slot + c_at(j, r),
                                        __builtin_fmaf(p.alpha_f, acc[i][j][r], p.beta_f * cv[j][r]));
                } else {
                    Out<OUT>::lds_store(slot + c_at(j, r), p.alpha_f * acc[i][j][r]);
                }
            }
        // the wave's LDS operations run in order: the reads below see the writes above
#pragma unroll
        for (int q = 0; q < L; ++q) {
            const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(slot + q * 1024 + 16 * lane);
            __builtin_amdgcn_raw_buffer_store_b128(v, rd, (int)chunk_off(i, q), 0,
                                                   kNT ? kStreamPolicy : 0);
        }
        if constexpr (kReadC && i + S < FM) {
            wait_lds<0>();                                  // the slot's values are in registers
            load_block_row(i + S, i % S);
        }
    });
}

// LDS bytes of one workgroup: the A and B stage buffers of 128 bytes per row (160 KB, all of
// a CU's LDS, at 256 x 256 with three B buffers)
template <int IN, int BM, int BN>
constexpr int tile_lds_bytes() {
    return (kBuffers * BM + b_buffers(IN) * BN) * kStageKBytes;
}

// ---------------------------------------------------------------------------------------
// One BM x BN tile of D (tile row tm, tile column tn) by one workgroup; smem holds at least
// tile_lds_bytes() of LDS.
// ---------------------------------------------------------------------------------------
template <int IN, int OUT, bool TA, bool TB, int BM, int BN, int NW>
__device__ __forceinline__ void gemm_tile(const Params &p, int tm, int tn, lds_char *smem) {
    constexpr bool kF8 = is_fp8(IN);
    static_assert(NW == 4 || (NW == 8 && !kF8), "4 waves, or 8 for 2-byte and INT8 inputs");
    constexpr int EB = (IN == IN_I8 || kF8) ? 1 : 2;
    constexpr int NSA = BM / 32, NSB = BN / 32;
    // 16-wide MFMA blocks per wave: a 2 x (NW / 2) wave grid
    constexpr int FM = BM / 32, FN = BN / (8 * NW);
    constexpr int kStageK = kStageKBytes / EB;
    using OpA = Operand<EB, !TA, NSA, NW / 4>;
    using OpB = Operand<EB, TB, NSB, NW / 4>;
    using acc_t = typename MmaAcc<IN>::type;
    constexpr int A_BYTES = OpA::kStageBytes, B_BYTES = OpB::kStageBytes;
    constexpr int kLoadsPerStage = OpA::kSlots + OpB::kSlots;   // per wave

    // LDS: [A stage 0 | A stage 1 | B stage 0 | B stage 1].  Stage parity is a compile-time
    // constant in the unrolled loop below, so every fragment read is one base register plus
    // an immediate offset.
    auto stage_a = [&](int parity) { return smem + parity * A_BYTES; };
    auto stage_b = [&](int parity) { return smem + kBuffers * A_BYTES + parity * B_BYTES; };

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    // With 8 waves, waves w and w + 4 (wm = 0 and 1) share a SIMD and a column of B blocks.
    const int wm = wave / (NW / 2), wn = wave % (NW / 2);
    const int vq = wave & 3, hi = wave >> 2;    // the quarter and position group it loads

    const int m0 = tm * BM, n0 = tn * BN;
    const int m_left = p.m - m0, n_left = p.n - n0;
    const bool full_mn = (m_left >= BM) && (n_left >= BN);

    OpA opa;
    OpB opb;
    opa.init(vq, hi, lane, p.lda, m_left, 0u);
    opb.init(vq, hi, lane, p.ldb, n_left, (uint32_t)(kBuffers * A_BYTES));

    const int nk = (p.k + kStageK - 1) / kStageK;
    const int k_tail = p.k % kStageK;

    // Stage cursors.  The guaranteed-readable end of an operand stored rows x cols with
    // leading dimension ld is the end of the 16-byte block holding its last element; the
    // last stage's record count is the distance from its start to that end.
    StageCursor ca, cb;
    {
        const int64_t ra = TA ? p.k : p.m, cla = TA ? p.m : p.k;
        const int64_t rb = TB ? p.n : p.k, clb = TB ? p.k : p.n;
        const int64_t end_a = (ra - 1) * p.lda * EB + ((cla * EB + 15) & ~(int64_t)15);
        const int64_t end_b = (rb - 1) * p.ldb * EB + ((clb * EB + 15) & ~(int64_t)15);
        const int64_t off_a = TA ? (int64_t)m0 * EB : (int64_t)m0 * p.lda * EB;
        const int64_t off_b = TB ? (int64_t)n0 * p.ldb * EB : (int64_t)n0 * EB;
        ca.step = TA ? (int64_t)kStageK * p.lda * EB : kStageKBytes;
        cb.step = TB ? kStageKBytes : (int64_t)kStageK * p.ldb * EB;
        ca.base = (uint64_t)p.A + (uint64_t)off_a;
        cb.base = (uint64_t)p.B + (uint64_t)off_b;
        const int64_t la = end_a - off_a - (int64_t)(nk - 1) * ca.step;
        const int64_t lb = end_b - off_b - (int64_t)(nk - 1) * cb.step;
        ca.last_records = (int)(la < 0 ? 0 : (la > kNumRecords ? kNumRecords : la));
        cb.last_records = (int)(lb < 0 ? 0 : (lb > kNumRecords ? kNumRecords : lb));
    }

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{};

    const uint32_t lds_w = (uint32_t)(uintptr_t)smem +
                           (uint32_t)__builtin_amdgcn_readfirstlane(hi * 4096 + vq * 1024);
    // K ends inside the last stage: its K-contiguous chunks past K are zeroed once they have
    // landed (wave-uniform test).  pa: the stage's A buffer; b_off: its B buffer's offset
    // from the first B buffer.
    auto fix_stage = [&](int s, int pa, uint32_t b_off) {
        if (k_tail != 0 && s == nk - 1) {
            wait_vmem<0>();  // this lane's chunks have landed
            opa.fix_k_tail(stage_a(pa), k_tail, vq, hi, lane);
            opb.fix_k_tail(stage_b(0) + b_off, k_tail, vq, hi, lane);
        }
    };

    if constexpr (!kF8) {
        // Fragment registers: two sets, one per k step of a stage.
        u32x4 fa[2][FM], fb[2][FN];
        constexpr int kMf = FM * FN, kUnits = FM + FN;
        // B's buffer offset changes every stage (three buffers against A's two), so its fragment
        // addresses are not immediates: at 128 x 128 per wave the kReadBases base registers of
        // the next stage's B buffer are set once per stage (set_bases, pinned in MFMA groups
        // with room for them), and each read is one of them plus an immediate.  Otherwise the
        // compiler adds the buffer offset beside each read, one instruction over a group's budget.
        constexpr bool kPinB = kMf >= 64 && (TB || FN % OpB::kGroupBlocks == 0);
        constexpr int kRB = OpB::kReadBases;
        uint32_t bb[2][kRB];
        const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
        auto set_base = [&](int par, uint32_t b_off, int i) {
            bb[par][i] = opb.read_base(smem_addr + b_off, i, wn * FN);
            asm volatile("" : "+v"(bb[par][i]));
        };
        // read unit u (< FM + FN) of k step ks: fragment u of A from A buffer pa, or fragment
        // u - FM of B from the B buffer at b_off (whose bases are bb[bpar])
        auto read_unit = [&](int set, int pa, uint32_t b_off, int bpar, int ks, int u) {
            if (u < FM) {
                fa[set][u] = opa.frag(smem + pa * A_BYTES, wm * FM + u, ks);
            } else {
                const int j = u - FM;
                if constexpr (kPinB)
                    fb[set][j] = opb.frag_at(bb[bpar][TB ? ks : j % OpB::kGroupBlocks], j, ks);
                else
                    fb[set][j] = opb.frag(smem + b_off, wn * FN + j, ks);
            }
        };
        // Load slot l of a stage's A (into A buffer pa) or B (into the B buffer whose LDS
        // address, plus this wave's quarter, is b_base); rs_a / rs_b address the stage.  b_base
        // passes through an empty statement at each load, so that each load's m0 is formed in its
        // own group rather than all of them ahead of the first.
        i32x4 rs_a, rs_b;
        auto load_a = [&](int pa, int l) { opa.load(rs_a, lds_w + (uint32_t)(pa * A_BYTES), l); };
        auto load_b = [&](uint32_t &b_base, int l) {
            asm volatile("" : "+s"(b_base));
            opb.load(rs_b, b_base, l);
        };
        // Prepare the resources of stage s (the cursors then move to stage s + 1).
        auto next_rsrc_a = [&](int s) { rs_a = ca.rsrc(s, nk); ca.advance(); keep_here(rs_a); keep_here(ca.base); };
        auto next_rsrc_b = [&](int s) { rs_b = cb.rsrc(s, nk); cb.advance(); keep_here(rs_b); keep_here(cb.base); };
        // In the loop the same resources are prepared in eight pieces of one or two scalar
        // instructions (for A, then B: the record count in two selects, the words, the
        // advance), each pinned in its own gap between MFMAs.
        int nr_a = 0, nr_b = 0;
        auto rsrc_piece = [&](auto p_c, int s) {
            constexpr int p = decltype(p_c)::value;
            StageCursor &c = p < 4 ? ca : cb;
            int &nr = p < 4 ? nr_a : nr_b;
            i32x4 &rs = p < 4 ? rs_a : rs_b;
            // The cursor passes through an empty statement first, so that the piece's
            // instructions are formed in its own group instead of being hoisted ahead of the step
            // (the stage index s arrives the same way, once per stage).
            if constexpr (p % 4 == 0) { nr = s == nk - 1 ? c.last_records : 0; keep_here(nr); }
            if constexpr (p % 4 == 1) { nr = s < nk - 1 ? kNumRecords : nr; keep_here(nr); }
            if constexpr (p % 4 == 2) { asm volatile("" : "+s"(c.base)); rs = c.words(nr); keep_here(rs); }
            if constexpr (p % 4 == 3) { asm volatile("" : "+s"(c.base)); c.advance(); keep_here(c.base); }
        };

        // One k step: the FM x FN MFMAs of fragment set `set`, each in its own fenced group with
        // at most two other instructions -- a wave issues one instruction per four cycles, so
        // more would hold back the next 16-cycle MFMA.  The fragments of the next k step (into
        // the other set) are read at the even MFMAs of the first half; `extra` places the
        // step's resource pieces and loads.
        auto k_step = [&](auto set_c, int rd_pa, uint32_t rd_b, int rd_bpar, int rd_ks, auto &&extra) {
            constexpr int set = decltype(set_c)::value;
            // The fragments of this k step were read during the first half of the previous one:
            // one wait for all of them instead of a wait before each MFMA that uses a new one.
            wait_lds<0>();
            static_for<kMf>([&](auto idx_c) {
                constexpr int idx = decltype(idx_c)::value;
                constexpr int i = idx / FN, j = idx % FN;
                Mma<IN>::run(fa[set][i], fb[set][j], acc[i][j]);
                extra(idx_c);
                static_for<kUnits>([&](auto u_c) {
                    constexpr int u = decltype(u_c)::value;
                    constexpr int at = 2 * kUnits <= kMf ? 2 * u : (u * kMf) / kUnits;
                    if constexpr (at == idx) read_unit(set ^ 1, rd_pa, rd_b, rd_bpar, rd_ks, u);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;

        // A stage's loads are split between its two k steps so that each carries half of them:
        // measured per k step, one that issues a whole stage's loads (16 per wave at 256 x 256)
        // runs at 64-85 % of the MFMA issue rate, one with half of them at 93 %, against 97 %
        // for one with none.  A is double-buffered and B triple-buffered (LDS:
        // [A 0 | A 1 | B 0 | B 1 | B 2]):
        //   k step 0 of stage s multiplies its first k half out of registers, reads the
        //     fragments of the second, and queues the B loads of stage s + 2 into the B buffer
        //     stage s - 1 has left (free since the barrier of stage s - 1);
        //   each wave then waits for its loads of stage s + 1 (the B loads just queued may stay
        //     in flight), and one barrier publishes stage s + 1 and certifies that every wave
        //     has read its last fragments of stage s;
        //   k step 1 multiplies the second k half, reads the first fragments of stage s + 1, and
        //     queues the A loads of stage s + 2 into the A buffer stage s has just left.
        // Every load has at least one k step to land before the barrier that waits for it; B's
        // (the operand whose loads land last on row-major NN products) have a stage and a half.
        // The resources of stage s + 2 are prepared in k step 0, a few scalar instructions at a
        // time: B's pieces first, at the first odd MFMAs, then B's loads at later odd MFMAs, and
        // A's pieces at even MFMAs past the fragment reads.  The B buffer offsets rotate by one
        // buffer per stage: b_cur (stage s), b_next (s + 1), b_load (s + 2).
        constexpr int kLoadsB = OpB::kSlots, kLoadsA = OpA::kSlots;
        uint32_t b_cur = 0, b_next = B_BYTES, b_load = 2 * B_BYTES;
        auto stage_iter = [&](int s, auto par_c) {
            constexpr int P = decltype(par_c)::value;
            uint32_t b_ld = lds_w + (uint32_t)(kBuffers * A_BYTES) + b_load;
            int s2 = s + 2;
            k_step(C0{}, P, b_cur, P, 1, [&](auto idx_c) {
                constexpr int idx = decltype(idx_c)::value;
                if constexpr (kMf >= 64) {
                    if constexpr (idx == 0) asm volatile("" : "+s"(s2));
                    // the LDS base of B's loads (formed here, from an opaque copy of the buffer
                    // offset), then the bases of the next stage's B reads
                    if constexpr (idx == 6) {
                        uint32_t bl = b_load;
                        asm volatile("" : "+s"(bl));
                        b_ld = lds_w + (uint32_t)(kBuffers * A_BYTES) + bl;
                        asm volatile("" : "+s"(b_ld));
                    }
                    if constexpr (kPinB) {
                        static_for<kRB>([&](auto i_c) {
                            if constexpr (idx == 2 * kUnits + 8 + 2 * decltype(i_c)::value)
                                set_base(P ^ 1, b_next, decltype(i_c)::value);
                        });
                    }
                    static_for<4>([&](auto q_c) {
                        constexpr int q = decltype(q_c)::value;
                        if constexpr (idx == 2 * q + 1)
                            rsrc_piece(std::integral_constant<int, 4 + q>{}, s2);
                        if constexpr (idx == 2 * kUnits + 2 * q)
                            rsrc_piece(std::integral_constant<int, q>{}, s2);
                    });
                    static_for<kLoadsB>([&](auto l_c) {
                        constexpr int l = decltype(l_c)::value;
                        constexpr int span = (kMf - 10) / 2;
                        constexpr int at = 9 + 2 * ((l * span) / (kLoadsB > 1 ? kLoadsB - 1 : 1));
                        if constexpr (at == idx) load_b(b_ld, l);
                    });
                } else {
                    // short k steps (smaller tiles): every piece beside the first MFMA
                    if constexpr (idx == 0) {
                        static_for<4>([&](auto q_c) { rsrc_piece(std::integral_constant<int, 4 + decltype(q_c)::value>{}, s + 2); });
                        static_for<4>([&](auto q_c) { rsrc_piece(q_c, s + 2); });
                    }
                    static_for<kLoadsB>([&](auto l_c) {
                        constexpr int l = decltype(l_c)::value;
                        if constexpr (((l * kMf) / kLoadsB + 1) % kMf == idx) load_b(b_ld, l);
                    });
                }
            });
            wait_vmem<kLoadsB>();  // this wave's loads of stage s + 1 have landed
            fix_stage(s + 1, P ^ 1, b_next);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            k_step(C1{}, P ^ 1, b_next, P ^ 1, 0, [&](auto idx_c) {
                constexpr int idx = decltype(idx_c)::value;
                static_for<kLoadsA>([&](auto l_c) {
                    constexpr int l = decltype(l_c)::value;
                    if constexpr (((l * kMf) / kLoadsA + 1) % kMf == idx) load_a(P, l);
                });
            });
            const uint32_t b_free = b_cur;
            b_cur = b_next;
            b_next = b_load;
            b_load = b_free;
        };

        // Prologue: stages 0 and 1 are queued; wait for stage 0.
        next_rsrc_a(0);
        next_rsrc_b(0);
        uint32_t b_ld0 = lds_w + (uint32_t)(kBuffers * A_BYTES);
        uint32_t b_ld1 = b_ld0 + (uint32_t)B_BYTES;
        static_for<kLoadsA>([&](auto l_c) { load_a(0, decltype(l_c)::value); });
        static_for<kLoadsB>([&](auto l_c) { load_b(b_ld0, decltype(l_c)::value); });
        next_rsrc_a(1);
        next_rsrc_b(1);
        static_for<kLoadsA>([&](auto l_c) { load_a(1, decltype(l_c)::value); });
        static_for<kLoadsB>([&](auto l_c) { load_b(b_ld1, decltype(l_c)::value); });
        if constexpr (kPinB)
            static_for<kRB>([&](auto i_c) { set_base(0, 0u, decltype(i_c)::value); });
        wait_vmem<kLoadsPerStage>();
        fix_stage(0, 0, 0);
        __syncthreads();
    #pragma unroll
        for (int u = 0; u < kUnits; ++u) read_unit(0, 0, 0, 0, 0, u);

        // Stages are taken in pairs (A buffer parity 0, then 1).  For an odd number of stages the
        // last pair's second stage lies past K: its loads read zero records, so it multiplies zeros
        // into the accumulators, which leaves them unchanged.
        for (int s = 0; s < nk; s += 2) {
            stage_iter(s, C0{});
            stage_iter(s + 1, C1{});
        }

    } else {
        // FP8: one v_mfma_f32_16x16x128_f8f6f4 per block and stage, on 8-dword fragments (the
        // stage's two 64-byte k steps as the two halves).  A stage runs in two halves around
        // its barrier: half 0 multiplies A blocks 0 .. HM-1, half 1 A blocks HM .. FM-1, each
        // against every B block, B-block-major.  With one register per fragment, each is
        // reloaded for the next use as soon as its last MFMA has issued: A blocks HM .. FM-1
        // of this stage during half 0; after the barrier has published the next stage, A blocks
        // 0 .. HM-1 at the start of half 1 and B block j right after its last MFMA in half 1.
        constexpr int HM = FM / 2;
        constexpr int kHalf = HM * FN;                 // MFMAs per half
        constexpr int kLastB = (FN - 1) * HM;          // half 0: first MFMA of the last B block
        constexpr int kReadsBeforeLastB = (2 * HM < (kLastB + 1) / 2) ? 2 * HM : (kLastB + 1) / 2;
        static_assert(FM % 2 == 0 && FN >= 2, "FP8 tiles");
        u32x8 fa8[FM], fb8[FN];
        auto read_a = [&](int parity, int blk, int ks) {
            set_half(fa8[blk], ks, opa.frag(smem + parity * A_BYTES, wm * FM + blk, ks));
        };
        // B from the B buffer at b_off (three buffers, rotating as in the 2-byte path)
        auto read_b = [&](uint32_t b_off, int blk, int ks) {
            set_half(fb8[blk], ks, opb.frag(smem + b_off, wn * FN + blk, ks));
        };
        i32x4 rs_a, rs_b;
        auto load_a = [&](int pa, int l) { opa.load(rs_a, lds_w + (uint32_t)(pa * A_BYTES), l); };
        auto load_b = [&](uint32_t b_off, int l) {
            opb.load(rs_b, lds_w + (uint32_t)(kBuffers * A_BYTES) + b_off, l);
        };
        constexpr int kLoadsB = OpB::kSlots, kLoadsA = OpA::kSlots;
        uint32_t b_cur = 0, b_next = B_BYTES, b_load = 2 * B_BYTES;
        auto next_rsrc_a = [&](int s) { rs_a = ca.rsrc(s, nk); ca.advance(); keep_here(rs_a); keep_here(ca.base); };
        auto next_rsrc_b = [&](int s) { rs_b = cb.rsrc(s, nk); cb.advance(); keep_here(rs_b); keep_here(cb.base); };
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;

        // Half 0 of stage s (A buffer P): the last B block's two reads (issued after the last
        // MFMA of the previous half 1) may still be in flight; they are waited for just before
        // that block's first MFMA, past the A reads this half has issued by then.  B's loads of
        // stage s + 2 go to the B buffer stage s - 1 left (its last reads, in half 1 of stage
        // s - 2, were certified by the barrier of stage s - 1); A's follow in half 1, so each half
        // carries half of a stage's loads.
        auto half0 = [&](int s, auto par_c) {
            constexpr int P = decltype(par_c)::value;
            wait_lds<2>();
            static_for<kHalf>([&](auto t_c) {
                constexpr int t = decltype(t_c)::value;
                constexpr int j = t / HM, i = t % HM;
                if constexpr (t == kLastB && kLastB > 0) wait_lds<kReadsBeforeLastB>();
                Mma8<IN>::run(fa8[i], fb8[j], acc[i][j]);
                if constexpr (t == 1 % kHalf) next_rsrc_a(s + 2);
                if constexpr (t == 3 % kHalf) next_rsrc_b(s + 2);
                static_for<2 * HM>([&](auto r_c) {     // A blocks HM .. FM-1 of this stage
                    constexpr int r = decltype(r_c)::value;
                    if constexpr (2 * r == t) read_a(P, HM + r / 2, r % 2);
                });
                static_for<kLoadsB>([&](auto l_c) {    // past the B resource (MFMA 3)
                    constexpr int l = decltype(l_c)::value;
                    constexpr int at = kHalf > 4 ? 4 + (l * (kHalf - 4)) / kLoadsB : (3 + l) % kHalf;
                    if constexpr (at == t) load_b(b_load, l);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // Half 1 of stage s: the next stage (A buffer P ^ 1, B buffer b_next) is in LDS; A's
        // loads of stage s + 2 go to A buffer P, which every wave has finished reading.
        auto half1 = [&](auto par_c) {
            constexpr int P = decltype(par_c)::value;
            wait_lds<0>();
            static_for<kHalf>([&](auto t_c) {
                constexpr int t = decltype(t_c)::value;
                constexpr int j = t / HM, i = HM + t % HM;
                Mma8<IN>::run(fa8[i], fb8[j], acc[i][j]);
                static_for<2 * HM>([&](auto r_c) {     // next stage: A blocks 0 .. HM-1
                    constexpr int r = decltype(r_c)::value;
                    if constexpr (r == t) read_a(P ^ 1, r / 2, r % 2);
                });
                static_for<FN>([&](auto jj_c) {        // next stage: B block jj after its last use
                    constexpr int jj = decltype(jj_c)::value;
                    if constexpr (t == (jj + 1) * HM - 1) {
                        read_b(b_next, jj, 0);
                        read_b(b_next, jj, 1);
                    }
                });
                static_for<kLoadsA>([&](auto l_c) {
                    constexpr int l = decltype(l_c)::value;
                    constexpr int at = ((l * kHalf) / kLoadsA + 1) % kHalf;
                    if constexpr (at == t) load_a(P, l);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        auto stage8 = [&](int s, auto par_c) {
            constexpr int P = decltype(par_c)::value;
            half0(s, par_c);
            wait_vmem<kLoadsB>();  // this wave's loads of stage s + 1 have landed
            fix_stage(s + 1, P ^ 1, b_next);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            half1(par_c);
            const uint32_t b_free = b_cur;
            b_cur = b_next;
            b_next = b_load;
            b_load = b_free;
        };

        // Prologue: stages 0 and 1 queued, stage 0 waited for; then the fragments half 0 of
        // stage 0 needs first (A blocks 0 .. HM-1, every B block; the last B block last).
        next_rsrc_a(0);
        next_rsrc_b(0);
        static_for<kLoadsA>([&](auto l_c) { load_a(0, decltype(l_c)::value); });
        static_for<kLoadsB>([&](auto l_c) { load_b(0, decltype(l_c)::value); });
        next_rsrc_a(1);
        next_rsrc_b(1);
        static_for<kLoadsA>([&](auto l_c) { load_a(1, decltype(l_c)::value); });
        static_for<kLoadsB>([&](auto l_c) { load_b(B_BYTES, decltype(l_c)::value); });
        wait_vmem<kLoadsPerStage>();
        fix_stage(0, 0, 0u);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2 * HM; ++r) read_a(0, r / 2, r % 2);
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
            read_b(0, jj, 0);
            read_b(0, jj, 1);
        }
        // once: the loop head then sees at most the last B block's reads of a half 1 pending
        wait_lds<0>();
        for (int s = 0; s < nk; s += 2) {
            stage8(s, C0{});
            stage8(s + 1, C1{});
        }
    }
    wait_vmem<0>();  // no direct load into LDS is left in flight when the workgroup ends
    drain_mfma(acc);

    // ---- epilogue
    // (full_mn, p.read_c and the wave index are uniform across a wave)
    // The lane index passes through an empty statement here, so that the epilogue's per-lane
    // addresses are computed after the loop rather than held in registers across it.
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    constexpr int kRegion = kBuffers * (A_BYTES + B_BYTES) / NW;  // LDS bytes per wave
    const int w = __builtin_amdgcn_readfirstlane(wave);
    lds_char *region = smem + w * kRegion;
    const uint32_t region_addr = (uint32_t)(uintptr_t)smem + (uint32_t)(w * kRegion);
    if (full_mn) {
        // every wave's loads and fragment reads are complete: the LDS is free
        __syncthreads();
        // C's loads and D's stores cover whole 128-byte lines when the row pitch and the
        // pointers are line-aligned: then they stream past the caches (non-temporal); partial
        // lines keep the default policy, under which the L2 gathers them
        constexpr int OB = Out<OUT>::kBytes;
        const bool lines = ((uint64_t)p.ldc * OB) % 128 == 0 &&
                           (((uintptr_t)p.D | (p.read_c ? (uintptr_t)p.C : 0)) & 127) == 0;
        if (p.read_c) {
            if (lines)
                store_full_tile_staged<IN == IN_I8, OUT, FM, FN, BM, BN, kRegion, NW, true, true>(
                    p, acc, m0, n0, wm, wn, lane_e, region, region_addr);
            else
                store_full_tile_staged<IN == IN_I8, OUT, FM, FN, BM, BN, kRegion, NW, true, false>(
                    p, acc, m0, n0, wm, wn, lane_e, region, region_addr);
        } else {
            if (lines)
                store_full_tile_staged<IN == IN_I8, OUT, FM, FN, BM, BN, kRegion, NW, false, true>(
                    p, acc, m0, n0, wm, wn, lane_e, region, region_addr);
            else
                store_full_tile_staged<IN == IN_I8, OUT, FM, FN, BM, BN, kRegion, NW, false, false>(
                    p, acc, m0, n0, wm, wn, lane_e, region, region_addr);
        }
    } else if (p.read_c) {
        __syncthreads();
        store_tile_c_staged<IN == IN_I8, OUT, FM, FN, BM, BN, kRegion, false, NW>(
            p, acc, m0, n0, wm, wn, lane_e, m_left, n_left, region, region_addr);
    } else {
        store_tile<IN == IN_I8, OUT, FM, FN, BM, BN, false, NW>(p, acc, m0, n0, wm, wn, lane_e,
                                                                m_left, n_left);
    }
}

// ---------------------------------------------------------------------------------------
// The kernel: one tile per workgroup.
// ---------------------------------------------------------------------------------------
template <int IN, int OUT, bool TA, bool TB, int BM, int BN, int NW = 4>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) char smem_raw[tile_lds_bytes<IN, BM, BN>()];
    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    gemm_tile<IN, OUT, TA, TB, BM, BN, NW>(p, tm, tn, (lds_char *)smem_raw);
}

// Host-side launcher of one instance.  hipLaunchKernel returns this launch's own status (an
// error the caller left pending on the thread is neither reported nor cleared).
template <int IN, int OUT, bool TA, bool TB, int BM, int BN, int NW = 4>
hipError_t launch(const Params &p, hipStream_t stream) {
    const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    void *args[] = {const_cast<Params *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_kernel<IN, OUT, TA, TB, BM, BN, NW>),
                           dim3(grid), dim3(NW * 64), args, 0, stream);
}

// Entry points of the per-input-type translation units.
hipError_t launch_f16(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_bf16(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_i8(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_fp8(int in, int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
// one FP8 format pair each (kern_fp8_*.hip)
hipError_t launch_fp8_fp8(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_fp8_bf8(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_bf8_fp8(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_bf8_bf8(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
// 2:4 structured-sparse A (sp24_kernel.inc; launcher in sp24.hip, instances in sp24_<type>.hip):
// A's kept values (m x k/2, lda) in Params::A, their indices (2 bits per kept value, in k order;
// m rows of ld_meta bytes) in meta.
struct SpParams {
    Params p;
    const void *meta;
    int64_t ld_meta;
};
hipError_t launch_sp24(int in, int out, bool tb, const SpParams &sp, hipStream_t stream);
// one input type each
hipError_t launch_sp24_f16(int out, bool tb, const SpParams &sp, hipStream_t stream);
hipError_t launch_sp24_bf16(int out, bool tb, const SpParams &sp, hipStream_t stream);
hipError_t launch_sp24_i8(int out, bool tb, const SpParams &sp, hipStream_t stream);
hipError_t launch_sp24_fp8_fp8(int out, bool tb, const SpParams &sp, hipStream_t stream);
hipError_t launch_sp24_fp8_bf8(int out, bool tb, const SpParams &sp, hipStream_t stream);
hipError_t launch_sp24_bf8_fp8(int out, bool tb, const SpParams &sp, hipStream_t stream);
hipError_t launch_sp24_bf8_bf8(int out, bool tb, const SpParams &sp, hipStream_t stream);
// BF16 pieces of an FP32 operand for the three-product GEMM (bf16x3.hip).
hipError_t launch_split_bf16x3(const float *in, int64_t rows, int64_t cols, int64_t ld_in,
                               void *out, int64_t ld_out, bool k_along_cols, int pieces,
                               hipStream_t stream);

}  // namespace mpg
