// sp24.hip -- GEMM with a 2:4 structured-sparse A on gfx950's sparse matrix cores:
//
//   D = alpha * A * op(B) + beta * C,   A: m x k with at most 2 nonzeros in every group of 4
//                                        consecutive k, given compressed (values + indices)
//
// Sparse tensor cores as the page "稀疏张量核心加速模板计算的技术解析" (sparse tensor cores
// for stencil computation) describes them in sections 1.2.1 and 1.3.2: a 2:4 sparse operand is
// held as its kept values (half of k) plus 2 bits of metadata per kept value (its position
// within its group of 4), and the matrix instruction skips the zeros.  Here the instructions
// are v_smfmac_f32_16x16x64_{f16,bf16} and v_smfmac_i32_16x16x128_i8: a 16 x 16 output block
// over one k step (64 logical k for 16-bit inputs, 128 for INT8) from A's kept values (lane
// group g: the 16 bytes of kept values of logical k 16 g .. 16 g + 15, resp. 32 g .. 32 g + 31),
// B's k-rows (the two dense fragments of the step's halves, 32 bytes) and an index register
// (2 bits per kept value, in k order: the low 16 bits for 16-bit inputs, all 32 for INT8) --
// lane layouts measured on gfx950.
//
// One sparse instruction does the useful work of one dense 16 x 16 x 32 in the same issue
// time, so per MFMA cycle the sparse loop needs about twice the bytes of the dense kernel.  The
// loop is therefore built around the global -> LDS stream:
//   * tile 256 x 256 (2 x 2 waves of 128 x 128), the largest the accumulators allow;
//   * a stage is one sparse k step: A's kept values, 64 bytes per row, and B's k-rows (the
//     dense kernel's B stage) -- 48 KB -- plus, every fourth (16-bit) or second (INT8) stage,
//     32 metadata bytes per row covering those stages (8 KB; two lanes per row, so one 32-byte
//     request per row: the loop is bound by the L2 request rate, not by bytes);
//   * an LDS ring of three stages (and two metadata quads), so that two stages of loads are in
//     flight while the third is multiplied: each iteration waits only for the older one;
//   * all fragments of the next stage are read during the current one; a B block's register
//     is refilled right after its last MFMA, and B block 7 alternates between two registers so
//     that its refill is not the last instruction of the iteration.
// LDS: [A ring 3 x 16 KB | B ring 3 x 32 KB | metadata 2 x 8 KB] = 160 KB.  k must be a
// multiple of 128 (whole stages, no K tail); m and n are arbitrary.
#include "mpgemm_kernel.hpp"

namespace mpg {

namespace {

template <int IN> struct SMma;
template <> struct SMma<IN_F16> {
    static __device__ __forceinline__ void run(u32x4 a, u32x8 b, uint32_t idx, f32x4 &c) {
        asm("v_smfmac_f32_16x16x64_f16 %0, %1, %2, %3" : "+a"(c) : "v"(a), "v"(b), "v"(idx));
    }
};
template <> struct SMma<IN_BF16> {
    static __device__ __forceinline__ void run(u32x4 a, u32x8 b, uint32_t idx, f32x4 &c) {
        asm("v_smfmac_f32_16x16x64_bf16 %0, %1, %2, %3" : "+a"(c) : "v"(a), "v"(b), "v"(idx));
    }
};
template <> struct SMma<IN_I8> {
    static __device__ __forceinline__ void run(u32x4 a, u32x8 b, uint32_t idx, i32x4 &c) {
        asm("v_smfmac_i32_16x16x128_i8 %0, %1, %2, %3" : "+a"(c) : "v"(a), "v"(b), "v"(idx));
    }
};

typedef __attribute__((address_space(3))) unsigned short lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// A's kept values, K-contiguous: a stage holds 256 rows of 64 bytes (row r at r * 64, its
// 16-byte chunk c at chunk position c ^ swz(r)).  A fragment read (16 rows x 64 bytes; lanes
// 0-31 take chunks 0-1 of rows 0-15, lanes 32-63 chunks 2-3) is served 32 lanes at a time over
// 128 four-byte banks: rows r and r + 8 share a bank base, so rows 8-15 swap chunk pairs.
struct KeptA {
    static constexpr int kRows = 256;
    static constexpr int kStageBytes = kRows * 64;     // 16 KB
    static constexpr int kSlots = kStageBytes / 4096;  // 1 KB loads per wave per stage
    uint32_t voff[kSlots];
    uint32_t r_off;
    static __device__ __forceinline__ int swz(int r) { return ((r >> 3) & 1) << 1; }
    // Load slot i of wave w, lane l fills LDS bytes i * 4096 + w * 1024 + l * 16 of the stage:
    // row 64 i + 16 w + l / 4, physical chunk l % 4.  Rows past the matrix repeat its last row.
    __device__ __forceinline__ void init(int wave, int lane, int64_t lda_bytes, int m_left) {
        const uint32_t row_bytes = (uint32_t)lda_bytes;
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int r = 64 * i + 16 * wave + lane / 4;
            const int c = (lane % 4) ^ swz(r);
            voff[i] = (uint32_t)min(r, m_left - 1) * row_bytes + 16u * (uint32_t)c;
        }
        const int u = lane % 16, g = lane / 16;
        r_off = (uint32_t)(u * 64 + 16 * (g ^ swz(u)));
    }
    __device__ __forceinline__ void load(i32x4 rs, uint32_t lds_stage_w, int i) const {
        dma16(rs, voff[i], 0u, lds_stage_w + (uint32_t)i * 4096u);
    }
    // 16-byte operand of 16-row block `blk` (the lane's row blk * 16 + lane % 16)
    __device__ __forceinline__ u32x4 frag(const lds_char *stage, int blk) const {
        return *(const lds_u32x4 *)(stage + blk * 1024 + r_off);
    }
};

}  // namespace

template <int IN, int OUT, bool TB>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void sp24_kernel(SpParams sp) {
    const Params &p = sp.p;
    constexpr int BM = kSpTileM, BN = kSpTileN;
    constexpr int FM = BM / 32, FN = BN / 32;       // 16-wide blocks per wave (2 x 2 waves)
    constexpr bool kInt = IN == IN_I8;
    constexpr int EB = kInt ? 1 : 2;                // bytes per element
    using OpB = Operand<EB, TB, BN / 32>;           // one stage of B: 64 (16-bit) or 128 k-rows
    using acc_t = typename MmaAcc<IN>::type;
    constexpr int kStageK = 128 / EB;               // logical k per stage: 64 kept bytes per row
    constexpr int kMetaStages = kInt ? 2 : 4;       // stages per 32-byte metadata row
    static_assert(OpB::kStageK == kStageK, "A and B stages cover the same k");
    constexpr int kRing = 3;
    constexpr int A_STAGE = KeptA::kStageBytes;     // 16 KB
    constexpr int B_STAGE = OpB::kStageBytes;       // 32 KB
    constexpr int M_QUAD = BM * 32;                 // metadata of four stages: 32 bytes per row
    constexpr int B_BASE = kRing * A_STAGE, M_BASE = B_BASE + kRing * B_STAGE;
    constexpr int kLoadsAB = KeptA::kSlots + OpB::kSlots;   // 12 per wave per stage
    constexpr int kLoadsM = M_QUAD / 4096;                  // + 2 metadata loads every 4th stage
    static_assert(FM == 8 && FN == 8, "tile");

    __shared__ __attribute__((aligned(16))) char smem_raw[M_BASE + 2 * M_QUAD];
    lds_char *smem = (lds_char *)smem_raw;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int m_left = p.m - m0, n_left = p.n - n0;
    const bool full_mn = (m_left >= BM) && (n_left >= BN);

    KeptA opa;
    OpB opb;
    opa.init(wave, lane, p.lda * EB, m_left);
    opb.init(wave, lane, p.ldb, n_left, 0u);
    const int nk = p.k / kStageK;                    // stages (k is a multiple of 128)
    const int nq = (nk + kMetaStages - 1) / kMetaStages;   // 32-byte metadata groups

    // Stage cursors: the exact readable end of each operand bounds its last stage.
    StageCursor ca, cb, cm;
    {
        const int64_t end_a = (int64_t)(p.m - 1) * p.lda * EB + (int64_t)p.k / 2 * EB;
        const int64_t rb = TB ? p.n : p.k, clb = TB ? p.k : p.n;
        const int64_t end_b = (rb - 1) * p.ldb * EB + ((clb * EB + 15) & ~(int64_t)15);
        const int64_t end_m = (int64_t)(p.m - 1) * sp.ld_meta + (int64_t)p.k / 8;
        const int64_t off_a = (int64_t)m0 * p.lda * EB;
        const int64_t off_b = TB ? (int64_t)n0 * p.ldb * EB : (int64_t)n0 * EB;
        const int64_t off_m = (int64_t)m0 * sp.ld_meta;
        ca.step = 64;
        cb.step = TB ? 128 : (int64_t)kStageK * p.ldb * EB;
        cm.step = 32;
        ca.base = (uint64_t)p.A + (uint64_t)off_a;
        cb.base = (uint64_t)p.B + (uint64_t)off_b;
        cm.base = (uint64_t)sp.meta + (uint64_t)off_m;
        auto last = [&](int64_t end, int64_t off, int64_t step, int count) {
            const int64_t l = end - off - (int64_t)(count > 0 ? count - 1 : 0) * step;
            return (int)(l < 0 ? 0 : (l > kNumRecords ? kNumRecords : l));
        };
        ca.last_records = last(end_a, off_a, ca.step, nk);
        cb.last_records = last(end_b, off_b, cb.step, nk);
        cm.last_records = last(end_m, off_m, cm.step, nq);
    }
    // metadata load i: lane l of wave w brings bytes 16 (l % 2) .. +15 of row
    // 128 i + 32 w + l / 2's quad (clamped to the last row) to LDS byte row * 32 + 16 (l % 2)
    uint32_t voff_m[kLoadsM];
#pragma unroll
    for (int i = 0; i < kLoadsM; ++i)
        voff_m[i] = (uint32_t)min(128 * i + 32 * wave + lane / 2, m_left - 1) * (uint32_t)sp.ld_meta +
                    16u * (uint32_t)(lane % 2);
    // metadata read: row wm * 128 + 16 i + lane % 16, lane group g's 8 (16-bit) or 16 (INT8)
    // positions: 2 or 4 bytes
    constexpr int kIdxBytes = kInt ? 4 : 2;
    const uint32_t m_lane = (uint32_t)((wm * (BM / 2) + lane % 16) * 32 + kIdxBytes * (lane / 16));

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{};

    const uint32_t lds_w = (uint32_t)(uintptr_t)smem + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
    i32x4 rs_a, rs_b, rs_m;
    // Resources of stage t (the cursors then move on); the metadata's for t a multiple of
    // kMetaStages.
    auto prep = [&](int t, auto meta_c) {
        rs_a = ca.rsrc(t, nk);
        ca.advance();
        rs_b = cb.rsrc(t, nk);
        cb.advance();
        if constexpr (decltype(meta_c)::value) {
            rs_m = cm.rsrc(t / kMetaStages, nq);
            cm.advance();
        }
    };
    // Load l of a stage into ring slot q (and metadata buffer mq): the metadata first when the
    // stage carries it, then A's slots, then B's.
    auto load_slot = [&](int q, int mq, auto meta_c, int l) {
        constexpr bool kMeta = decltype(meta_c)::value;
        if (kMeta && l < kLoadsM) {
            dma16(rs_m, voff_m[l], 0u, lds_w + (uint32_t)(M_BASE + mq * M_QUAD + l * 4096));
            return;
        }
        const int la = l - (kMeta ? kLoadsM : 0);
        if (la < KeptA::kSlots)
            opa.load(rs_a, lds_w + (uint32_t)(q * A_STAGE), la);
        else
            opb.load(rs_b, lds_w + (uint32_t)(B_BASE + q * B_STAGE), la - KeptA::kSlots);
    };

    // Fragments: A and the indices in two sets (this stage's, the next one's), B blocks 0-6 in
    // one register each (refilled after their last use), B block 7 in two alternating ones.
    u32x4 fa[2][FM];
    uint32_t fi[2][FM];
    u32x8 fb[FN - 1];
    u32x8 fb7[2];
    auto read_a = [&](int set, const lds_char *st, int i) { fa[set][i] = opa.frag(st, wm * FM + i); };
    // positions of stage part `part` (the stage's index within its metadata group)
    auto read_i = [&](int set, const lds_char *mst, int part, int i) {
        if constexpr (kInt)
            fi[set][i] = *(const lds_u32 *)(mst + m_lane + i * 512 + 16 * part);
        else
            fi[set][i] = *(const lds_u16 *)(mst + m_lane + i * 512 + 8 * part);
    };
    auto read_b = [&](u32x8 &dst, const lds_char *st, int j) {
        set_half(dst, 0, opb.frag(st, wn * FN + j, 0));
        set_half(dst, 1, opb.frag(st, wn * FN + j, 1));
    };

    // Prologue: stages 0, 1, 2 queued (metadata group 0 with stage 0, group 1 with stage 2
    // when groups are pairs); wait for stage 0 and read its fragments.
    using CT = std::integral_constant<bool, true>;
    using CF = std::integral_constant<bool, false>;
    using CM2 = std::integral_constant<bool, kMetaStages == 2>;
    constexpr int kLoads2 = kLoadsAB + (kMetaStages == 2 ? kLoadsM : 0);
    prep(0, CT{});
    static_for<kLoadsAB + kLoadsM>([&](auto l_c) { load_slot(0, 0, CT{}, decltype(l_c)::value); });
    prep(1, CF{});
    static_for<kLoadsAB>([&](auto l_c) { load_slot(1, 0, CF{}, decltype(l_c)::value); });
    prep(2, CM2{});
    static_for<kLoads2>([&](auto l_c) { load_slot(2, 1, CM2{}, decltype(l_c)::value); });
    wait_vmem<kLoadsAB + kLoads2>();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        read_a(0, smem, i);
        read_i(0, smem + M_BASE, 0, i);
    }
#pragma unroll
    for (int j = 0; j < FN - 1; ++j) read_b(fb[j], smem + B_BASE, j);
    read_b(fb7[0], smem + B_BASE, FN - 1);
    wait_lds<0>();

    // Iteration s (S4 = s % 4, H = s & 1) multiplies stage s (ring slot q) out of registers,
    // reads the fragments of stage s + 1 (ring slot q + 1) and queues the loads of stage s + 3
    // into slot q, whose last reads were waited for at the barrier.  Its first instructions wait
    // for stage s + 1 (at most one stage's loads, 12, may still be in flight: those of stage
    // s + 2, which has 14 when it carries metadata, so its two first loads are waited for too).
    auto iteration = [&](int s, int q, auto s4_c) {
        constexpr int S4 = decltype(s4_c)::value, H = S4 & 1;
        constexpr bool kMeta = (S4 + 3) % kMetaStages == 0;   // stage s + 3 starts a group
        constexpr int kL = kLoadsAB + (kMeta ? kLoadsM : 0);
        const int qn = q == kRing - 1 ? 0 : q + 1;
        wait_vmem<kLoadsAB>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        const lds_char *stA = smem + qn * A_STAGE;
        const lds_char *stB = smem + B_BASE + qn * B_STAGE;
        const lds_char *stM = smem + M_BASE + (((s + 1) / kMetaStages) & 1) * M_QUAD;
        const int mq = ((s + 3) / kMetaStages) & 1;
        static_for<FM * FN>([&](auto idx_c) {
            constexpr int idx = decltype(idx_c)::value;
            constexpr int j = idx / FM, i = idx % FM;   // B-block-major
            if constexpr (j < FN - 1)
                SMma<IN>::run(fa[H][i], fb[j], fi[H][i], acc[i][j]);
            else
                SMma<IN>::run(fa[H][i], fb7[H], fi[H][i], acc[i][j]);
            if constexpr (idx == 0) prep(s + 3, std::integral_constant<bool, kMeta>{});
            if constexpr (idx == 1) read_b(fb7[H ^ 1], stB, FN - 1);
            if constexpr (i == 2) read_a(H ^ 1, stA, j);
            if constexpr (i == 3) read_i(H ^ 1, stM, (S4 + 1) % kMetaStages, j);
            if constexpr (i == FM - 1 && j < FN - 1) read_b(fb[j], stB, j);
            static_for<kL>([&](auto l_c) {
                constexpr int l = decltype(l_c)::value;
                constexpr int at = 4 + (l * 58) / kL;
                if constexpr (at == idx) load_slot(q, mq, std::integral_constant<bool, kMeta>{}, l);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    auto next_q = [](int x) { return x == kRing - 1 ? 0 : x + 1; };
    int q = 0, s = 0;
    for (; s + 4 <= nk; s += 4) {
        iteration(s, q, C0{});
        q = next_q(q);
        iteration(s + 1, q, C1{});
        q = next_q(q);
        iteration(s + 2, q, C2{});
        q = next_q(q);
        iteration(s + 3, q, C3{});
        q = next_q(q);
    }
    // The remaining 1-3 stages, in pairs: a stage past K reads zero records for all its
    // operands, so it multiplies zeros into the accumulators, which leaves them unchanged.
    if (s < nk) {
        iteration(s, q, C0{});
        q = next_q(q);
        iteration(s + 1, q, C1{});
        q = next_q(q);
        if (s + 2 < nk) {
            iteration(s + 2, q, C2{});
            q = next_q(q);
            iteration(s + 3, q, C3{});
        }
    }
    wait_vmem<0>();  // no direct load into LDS is left in flight when the workgroup ends
    drain_mfma(acc);
    store_tile<kInt, OUT, FM, FN, BM, BN>(p, acc, m0, n0, wm, wn, lane, full_mn, m_left, n_left);
}

template __global__ void sp24_kernel<IN_F16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, true>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, true>(SpParams);
template __global__ void sp24_kernel<IN_I8, OUT_I32, false>(SpParams);
template __global__ void sp24_kernel<IN_I8, OUT_I32, true>(SpParams);

namespace {
template <int IN, int OUT, bool TB>
hipError_t launch_sp(const SpParams &sp, hipStream_t s) {
    const unsigned grid = (unsigned)sp.p.tiles_m * (unsigned)sp.p.tiles_n;
    hipLaunchKernelGGL((sp24_kernel<IN, OUT, TB>), dim3(grid), dim3(kThreads), 0, s, sp);
    return hipGetLastError();
}
template <int IN, int OUT>
hipError_t by_layout(bool tb, const SpParams &sp, hipStream_t s) {
    return tb ? launch_sp<IN, OUT, true>(sp, s) : launch_sp<IN, OUT, false>(sp, s);
}
}  // namespace

hipError_t launch_sp24(int in, int out, bool tb, const SpParams &sp, hipStream_t s) {
    if (in == IN_F16 && out == OUT_F32) return by_layout<IN_F16, OUT_F32>(tb, sp, s);
    if (in == IN_F16 && out == OUT_F16) return by_layout<IN_F16, OUT_F16>(tb, sp, s);
    if (in == IN_BF16 && out == OUT_F32) return by_layout<IN_BF16, OUT_F32>(tb, sp, s);
    if (in == IN_BF16 && out == OUT_BF16) return by_layout<IN_BF16, OUT_BF16>(tb, sp, s);
    if (in == IN_I8 && out == OUT_I32) return by_layout<IN_I8, OUT_I32>(tb, sp, s);
    return hipErrorInvalidValue;
}

}  // namespace mpg
