// mpgemm_kernel.hpp -- the gfx950 MFMA GEMM kernel: D = alpha * op(A) * op(B) + beta * C.
//
// One workgroup of 4 waves (256 lanes) computes a BM x BN tile of D.  The waves form a 2 x 2
// grid; each owns a (BM/2) x (BN/2) sub-tile made of 32 x 32 MFMA blocks whose accumulators
// stay in registers for the whole K loop.  K is walked in stages of 128 bytes per row (64
// FP16/BF16 elements or 128 INT8 elements): each stage is copied from global memory into one
// of two LDS buffers while the waves multiply out of the other one.
//
// The structure follows the pages' description of a tensor-core GEMM, re-planned for CDNA4:
//   * the product is a sum of rank-k slabs, each slab an outer product of a column panel of
//     A and a row panel of B ("The CUDA Handbook" section 17.5 "Tensor Cores", Figure 17-4);
//   * slabs are staged in on-chip shared memory in a block tile, each wave multiplying
//     fragments of it ("The CUDA Handbook" section 17.5, Listing 17-5 and the paragraph after
//     it, which also observes that the wait for the next slab's global load becomes the
//     bottleneck -- hence the double buffer here);
//   * the accumulator starts at zero, the K loop accumulates in place, and the epilogue scales
//     the product by alpha and adds beta * C element by element before storing
//     ("Programming Tensor Cores in CUDA 9", sections "Inner loop" and "Finishing");
//   * FP16/BF16 products are accumulated in FP32, INT8 products in INT32 ("Programming Tensor
//     Cores in CUDA 9", "What are Tensor Cores?"; "Mixed-Precision Programming with CUDA 8",
//     DP4A, Figure 2).
//
// MFMA lane layouts used (v_mfma_f32_32x32x16_{f16,bf16}, v_mfma_i32_32x32x32_i8): every
// operand register set is 16 bytes per lane; lane l holds row (A) or column (B) l % 32 and the
// 16-byte k chunk l / 32 of the 32-byte k step.  Accumulator register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l % 32 of the 32 x 32 block.
//
// LDS layout.  Each operand tile is a row of 4 KB sub-tiles, one per 32-row (A) or
// 32-column (B) MFMA block, so that every fragment address differs between blocks only by an
// immediate offset.
//   * K-contiguous operand (A with transa = N, B with transb = T): sub-tile = 32 rows x 128 B.
//     16-byte chunk c of row r sits at chunk position c ^ s(r), s(r) = (r & 7) ^ ((r >> 3) & 1),
//     so that the 32 rows of a ds_read_b128 spread over all banks for both 8- and 16-lane
//     LDS cycles.
//   * MN-contiguous operand (A with transa = T, B with transb = N): the tile keeps its global
//     orientation (k rows, 32 elements of m or n per sub-tile row: 64 B for 16-bit, 32 B for
//     8-bit types) and is transposed on the way out of LDS by ds_read_b64_tr_b16 /
//     ds_read_b64_tr_b8.  Within a 16-lane group these return, to lane t, element s of the
//     row read by lane 4s + t/4 (b16) or 2s + t/8 (b8), at position t % 4 (t % 8) of that row.
//     Chunk c of k-row k sits at c ^ L(k): L(k) = 2 * ((k >> 1) & 1) for 16-bit types,
//     (k >> 2) & 1 for 8-bit types.
//
// Edges: full tiles and full K stages take an unchecked path; a tile that crosses m or n, or
// the last stage when K is not a multiple of the stage, takes the checked path (a wave-uniform
// branch inside the same kernel).  Out-of-range chunks are fetched with a buffer offset
// beyond the resource's range, which the hardware returns as zero; a chunk that straddles K
// has its elements past K zeroed, so both operands are exactly zero beyond K and no NaN can
// leak in from padding.  Stores outside m x n are dropped the same way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) char lds_char;

enum InKind { IN_F16 = 0, IN_BF16 = 1, IN_I8 = 2 };
enum OutKind { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2, OUT_I32 = 3 };

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

constexpr int kThreads = 256;
constexpr int kStageKBytes = 128;   // bytes of k per row per stage
constexpr int kSubTileBytes = 4096; // 32 rows x 128 B, or the transposed equivalent
constexpr int kGroupM = 4;          // tile-row grouping for L2 reuse
constexpr uint32_t kOobOffset = 0x80000000u;  // a buffer offset past every resource's range
constexpr int kNumRecords = 0x7FFFFFFF;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    // raw buffer, stride 0; dword3 selects 32-bit data format (required non-zero on gfx9)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, kNumRecords,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
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
// Operand tile: global -> registers -> LDS copy, and LDS -> MFMA fragment reads.
//   EB: element bytes (2 or 1).  KC: K-contiguous storage.  NS: number of 32-wide sub-tiles.
// ---------------------------------------------------------------------------------------
template <int EB, bool KC, int NS>
struct Operand {
    static constexpr int kTileBytes = NS * kSubTileBytes;
    static constexpr int kChunkElems = 16 / EB;             // elements per 16-byte chunk
    static constexpr int kStageK = kStageKBytes / EB;       // k elements per stage
    // MN-contiguous geometry
    static constexpr int kRowBytes = 32 * EB;               // one k-row of a sub-tile
    static constexpr int kChunksPerRow = kRowBytes / 16;    // 4 (16-bit) or 2 (8-bit)
    static constexpr int kLanesPerSub = 64 / NS;            // lanes per sub-tile per load
    static constexpr int kRowsPerLoad = kLanesPerSub / kChunksPerRow;
    static_assert(NS == 2 || NS == 4 || NS == 8, "sub-tile count");

    // Per-thread copy state.
    uint32_t g_off0;    // global byte offset of slot 0, relative to the stage base
    uint32_t g_slot;    // global byte stride between slots
    uint32_t l_off0;    // LDS byte offset of slot 0 within the operand tile
    int mn0_idx;        // slot-0 index along m/n within the tile (K-contig: row; MN: chunk start)
    int k0_idx;         // slot-0 index along k within the stage (K-contig: chunk start; MN: row)
    uint32_t r_off[4];  // fragment read offsets (K-contig: one per k step; MN: one, plus steps)

    static constexpr uint32_t kLdsSlot = KC ? kSubTileBytes : 4u * kRowsPerLoad * kRowBytes;

    __device__ __forceinline__ void init(int wave, int lane, int64_t ld) {
        const uint32_t row_bytes = (uint32_t)(ld * EB);
        if constexpr (KC) {
            const int r = wave * 8 + lane / 8;                      // row within sub-tile 0
            const int c = (lane % 8) ^ (lane / 8) ^ (wave & 1);     // logical chunk
            mn0_idx = r;
            k0_idx = c * kChunkElems;
            g_off0 = (uint32_t)r * row_bytes + 16u * c;
            g_slot = 32u * row_bytes;
            l_off0 = (uint32_t)(wave * 1024 + lane * 16);
            // fragment reads: lane reads row lane%32, chunk 2*kk + lane/32, swizzled
            const int rr = lane % 32;
            const int sw = (rr & 7) ^ ((rr >> 3) & 1);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                r_off[kk] = (uint32_t)(rr * 128 + 16 * ((2 * kk + lane / 32) ^ sw));
        } else {
            const int st = lane / kLanesPerSub;
            const int within = lane % kLanesPerSub;
            const int kr = wave * kRowsPerLoad + within / kChunksPerRow;  // k-row of slot 0
            const int phys = within % kChunksPerRow;
            const int L = (EB == 2) ? 2 * ((kr >> 1) & 1) : ((kr >> 2) & 1);
            const int c = phys ^ L;
            mn0_idx = st * 32 + c * kChunkElems;
            k0_idx = kr;
            g_off0 = (uint32_t)kr * row_bytes + (uint32_t)(st * kRowBytes + 16 * c);
            g_slot = 4u * kRowsPerLoad * row_bytes;
            l_off0 = (uint32_t)(st * kSubTileBytes + kr * kRowBytes + 16 * phys);
            // transposed fragment reads (h = 0 half; steps add immediates)
            const int g = lane / 16, u = lane % 16;
            if constexpr (EB == 2) {
                const int k = 8 * (g >> 1) + (u >> 2);
                const int cc = 2 * (g & 1) + ((u & 3) >> 1);
                const int Lr = 2 * ((u >> 3) & 1);
                r_off[0] = (uint32_t)(k * kRowBytes + 16 * (cc ^ Lr) + 8 * (u & 1));
            } else {
                const int k = 16 * (g >> 1) + (u >> 1);
                const int cc = g & 1;
                const int Lr = (u >> 3) & 1;
                r_off[0] = (uint32_t)(k * kRowBytes + 16 * (cc ^ Lr) + 8 * (u & 1));
            }
            r_off[1] = r_off[2] = r_off[3] = 0;
        }
    }

    // Per-tile validity of this thread's chunks along m/n: K-contiguous chunks are valid for
    // slots below `slots_ok`; MN-contiguous chunks are all valid or all invalid.
    int slots_ok;

    __device__ __forceinline__ void set_tile(int mn_left) {
        if constexpr (KC) {
            const int rows = mn_left - mn0_idx;  // valid rows at or after slot 0's row
            slots_ok = rows <= 0 ? 0 : min(NS, (rows + 31) / 32);
        } else {
            slots_ok = mn0_idx < mn_left ? NS : 0;
        }
    }

    // Fetch this thread's NS chunks of one stage; `base` is the stage's start in global memory
    // and k_left the number of valid k elements from the stage start (<= 0 past the end).
    // Invalid chunks are fetched from beyond the buffer resource's range and arrive as zero.
    __device__ __forceinline__ void fetch(const char *base, u32x4 (&v)[NS], int k_left) const {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
        if constexpr (KC) {
            const bool k_ok = k_left - k0_idx > 0;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const uint32_t voff = (k_ok && i < slots_ok) ? g_off0 : kOobOffset;
                v[i] = buf_load16(rs, voff, i * g_slot);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const bool ok = i < slots_ok && k0_idx + i * 4 * kRowsPerLoad < k_left;
                v[i] = buf_load16(rs, ok ? g_off0 : kOobOffset, i * g_slot);
            }
        }
    }

    // K-contiguous chunks that straddle K get their elements past K zeroed (only ever needed
    // in the last stage; the caller branches on that, uniformly).
    __device__ __forceinline__ void mask_k_tail(u32x4 (&v)[NS], int k_left) const {
        if constexpr (KC) {
            const int nbytes = min(max(k_left - k0_idx, 0), kChunkElems) * EB;
#pragma unroll
            for (int i = 0; i < NS; ++i) v[i] = keep_first_bytes(v[i], nbytes);
        }
    }

    // Write the fetched chunks to LDS.
    __device__ __forceinline__ void stash(lds_char *tile, const u32x4 (&v)[NS]) const {
#pragma unroll
        for (int i = 0; i < NS; ++i)
            *(__attribute__((address_space(3))) u32x4 *)(tile + l_off0 + i * kLdsSlot) = v[i];
    }

    // 16-byte MFMA operand for 32-wide block `blk` at k step `kk` (0..3).
    __device__ __forceinline__ u32x4 frag(const lds_char *tile, int blk, int kk) const {
        if constexpr (KC) {
            return *(const __attribute__((address_space(3))) u32x4 *)(tile + blk * kSubTileBytes + r_off[kk]);
        } else if constexpr (EB == 2) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const lds_char *p = tile + blk * kSubTileBytes + r_off[0] + kk * 16 * kRowBytes;
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * kRowBytes));
            u32x4 r;
            r[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            r[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            r[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            r[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
            return r;
        } else {
            typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
            const lds_char *p = tile + blk * kSubTileBytes + r_off[0] + kk * 32 * kRowBytes;
            i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p));
            i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p + 8 * kRowBytes));
            u32x4 r;
            r[0] = (uint32_t)lo[0];
            r[1] = (uint32_t)lo[1];
            r[2] = (uint32_t)hi[0];
            r[3] = (uint32_t)hi[1];
            return r;
        }
    }
};

// ---------------------------------------------------------------------------------------
// MFMA per input type
// ---------------------------------------------------------------------------------------
template <int IN> struct Mma;
template <> struct Mma<IN_F16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(u32x4 a, u32x4 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mma<IN_BF16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(u32x4 a, u32x4 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mma<IN_I8> {
    typedef i32x16 acc_t;
    static __device__ __forceinline__ acc_t run(u32x4 a, u32x4 b, acc_t c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------------------
// Epilogue element: v = alpha * acc + beta * c, converted to the output type.
// ---------------------------------------------------------------------------------------
template <int OUT> struct Out;
template <> struct Out<OUT_F32> {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
    }
};
template <> struct Out<OUT_F16> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
        // v_cvt_f16_f32: round to nearest even under the default mode
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (_Float16)v), r, (int)off, 0, 0);
    }
};
template <> struct Out<OUT_BF16> {
    static constexpr int kBytes = 2;
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
    static __device__ __forceinline__ int load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, int v) {
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, r, (int)off, 0, 0);
    }
};

// Instruction interleaving hints for one stage (sched_group_barrier masks: 0x008 MFMA,
// 0x100 LDS read, 0x020 global read).  Before the barrier: k steps 0..2, each step's MFMAs
// with the next step's fragment reads spread over its first half and the next stage's global
// loads spread over step 0 (the LDS writes of the next stage follow).  After the barrier:
// k step 3 with the next stage's first fragment reads.
template <int I, int N, int W, int R, int L>
__device__ __forceinline__ void sched_interleave() {
    if constexpr (I < N) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (I < W) {
            constexpr int r = (R * (I + 1)) / W - (R * I) / W;
            constexpr int l = (L * (I + 1)) / W - (L * I) / W;
            if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
            if constexpr (l > 0) __builtin_amdgcn_sched_group_barrier(0x020, l, 0);
        }
        sched_interleave<I + 1, N, W, R, L>();
    }
}

template <int NMFMA, int NREAD, int NLOAD>
struct Sched {
    static constexpr int W = NMFMA > 1 ? NMFMA / 2 : 1;
    static __device__ __forceinline__ void compute() {
        sched_interleave<0, NMFMA, NMFMA, NREAD, NLOAD>();
        sched_interleave<0, NMFMA, W, NREAD, 0>();
        sched_interleave<0, NMFMA, W, NREAD, 0>();
    }
    static __device__ __forceinline__ void after_barrier() {
        sched_interleave<0, NMFMA, W, NREAD, 0>();
    }
};

// Map a workgroup id to its (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the 8 XCDs; ids are first remapped so that each XCD receives a contiguous run of tiles,
// and runs are laid out in groups of kGroupM tile-rows so that the tiles of one XCD share A
// row panels and B column panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int &tm, int &tn) {
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
// The kernel
// ---------------------------------------------------------------------------------------
template <int IN, int OUT, bool TA, bool TB, int BM, int BN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(Params p) {
    constexpr int EB = (IN == IN_I8) ? 1 : 2;
    constexpr int NSA = BM / 32, NSB = BN / 32;
    constexpr int FM = NSA / 2, FN = NSB / 2;   // MFMA blocks per wave (2 x 2 wave grid)
    constexpr int kStageK = kStageKBytes / EB;
    using OpA = Operand<EB, !TA, NSA>;
    using OpB = Operand<EB, TB, NSB>;
    using acc_t = typename Mma<IN>::acc_t;
    constexpr int A_BYTES = OpA::kTileBytes, B_BYTES = OpB::kTileBytes;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // LDS read instructions per k step: one per K-contiguous fragment, two per transposed one
    constexpr int kReadsPerStep = FM * (TA ? 2 : 1) + FN * (TB ? 1 : 2);

    __shared__ __attribute__((aligned(16))) char smem_raw[2 * STAGE_BYTES];
    lds_char *smem = (lds_char *)smem_raw;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int m_left = p.m - m0, n_left = p.n - n0;
    const bool full_mn = (m_left >= BM) && (n_left >= BN);

    OpA opa;
    OpB opb;
    opa.init(wave, lane, p.lda);
    opb.init(wave, lane, p.ldb);

    // Start of this tile's operand panels (bytes); stage s adds s * stage_step.
    const char *a_panel = (const char *)p.A + (TA ? (int64_t)m0 * EB : (int64_t)m0 * p.lda * EB);
    const char *b_panel = (const char *)p.B + (TB ? (int64_t)n0 * p.ldb * EB : (int64_t)n0 * EB);
    const int64_t a_step = TA ? (int64_t)kStageK * p.lda * EB : kStageKBytes;
    const int64_t b_step = TB ? kStageKBytes : (int64_t)kStageK * p.ldb * EB;

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{};

    const int nk = (p.k + kStageK - 1) / kStageK;
    u32x4 va[NSA], vb[NSB];

    opa.set_tile(m_left);
    opb.set_tile(n_left);
    auto fetch_stage = [&](int s) {
        const int k_left = p.k - s * kStageK;
        opa.fetch(a_panel + s * a_step, va, k_left);
        opb.fetch(b_panel + s * b_step, vb, k_left);
    };
    auto stash_stage = [&](int s, int buf) {
        const int k_left = p.k - s * kStageK;
        if (k_left < kStageK) {  // wave-uniform: the partial last stage, or past the end
            opa.mask_k_tail(va, k_left);
            opb.mask_k_tail(vb, k_left);
        }
        opa.stash(smem + buf * STAGE_BYTES, va);
        opb.stash(smem + buf * STAGE_BYTES + A_BYTES, vb);
    };

    // Fragment registers: two sets, so the reads of one k step overlap the MFMAs of another.
    u32x4 fa[2][FM], fb[2][FN];
    auto read_frags = [&](int set, const lds_char *tile, int kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[set][i] = opa.frag(tile, wm * FM + i, kk);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[set][j] = opb.frag(tile + A_BYTES, wn * FN + j, kk);
    };
    auto mfmas = [&](int set) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = Mma<IN>::run(fa[set][i], fb[set][j], acc[i][j]);
    };

    if (nk > 0) {
        fetch_stage(0);
        stash_stage(0, 0);
    }
    __syncthreads();
    read_frags(0, smem, 0);

    // Stage s multiplies out of LDS buffer s % 2 while stage s + 1 is fetched into registers
    // and written to the other buffer.  The one barrier per stage sits between k steps 2 and
    // 3: by then every wave has read its last fragments of buffer s % 2 and written stage
    // s + 1, so k step 3 can run while the first fragments of stage s + 1 are read.
    for (int s = 0; s < nk; ++s) {
        const lds_char *tcur = smem + (s & 1) * STAGE_BYTES;
        const lds_char *tnxt = smem + ((s & 1) ^ 1) * STAGE_BYTES;
        fetch_stage(s + 1);  // past the last stage every chunk is out of range: no traffic
        read_frags(1, tcur, 1);
        mfmas(0);
        read_frags(0, tcur, 2);
        mfmas(1);
        read_frags(1, tcur, 3);
        mfmas(0);
        Sched<FM * FN, kReadsPerStep, NSA + NSB>::compute();
        stash_stage(s + 1, (s & 1) ^ 1);
        __syncthreads();
        read_frags(0, tnxt, 0);
        mfmas(1);
        Sched<FM * FN, kReadsPerStep, NSA + NSB>::after_barrier();
    }

    // ---- epilogue: D = alpha * acc + beta * C, masked to m x n
    constexpr int OB = Out<OUT>::kBytes;
    const int64_t tile_off = ((int64_t)m0 * p.ldc + n0) * OB;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char *)p.D + tile_off);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const char *)(p.read_c ? p.C : p.D) + tile_off);
    const uint32_t ldc_b = (uint32_t)(p.ldc * OB);
    const int row_base = wm * (BM / 2) + 4 * (lane / 32);
    const int col_base = wn * (BN / 2) + (lane % 32);
    // byte offset of accumulator element r of block (i, j), or an out-of-range offset
    auto out_off = [&](int i, int j, int r) -> uint32_t {
        const int row = row_base + i * 32 + 8 * (r / 4) + (r % 4);
        const int col = col_base + j * 32;
        const bool ok = full_mn || (row < m_left && col < n_left);
        return ok ? (uint32_t)row * ldc_b + (uint32_t)col * OB : kOobOffset;
    };
    if (p.read_c) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                decltype(Out<OUT>::load(rc, 0)) cv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) cv[r] = Out<OUT>::load(rc, out_off(i, j, r));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if constexpr (IN == IN_I8) {
                        const uint32_t v = (uint32_t)p.alpha_i * (uint32_t)acc[i][j][r] +
                                           (uint32_t)p.beta_i * (uint32_t)cv[r];
                        Out<OUT>::store(rd, out_off(i, j, r), (int)v);
                    } else {
                        Out<OUT>::store(rd, out_off(i, j, r), p.alpha_f * acc[i][j][r] + p.beta_f * cv[r]);
                    }
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if constexpr (IN == IN_I8)
                        Out<OUT>::store(rd, out_off(i, j, r), (int)((uint32_t)p.alpha_i * (uint32_t)acc[i][j][r]));
                    else
                        Out<OUT>::store(rd, out_off(i, j, r), p.alpha_f * acc[i][j][r]);
                }
    }
}

// Host-side launcher of one instance.
template <int IN, int OUT, bool TA, bool TB, int BM, int BN>
hipError_t launch(const Params &p, hipStream_t stream) {
    const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    hipLaunchKernelGGL((gemm_kernel<IN, OUT, TA, TB, BM, BN>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// Entry points of the per-input-type translation units.
hipError_t launch_f16(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_bf16(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);
hipError_t launch_i8(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s);

}  // namespace mpg
