// sp24.hip -- GEMM with a 2:4 structured-sparse A on gfx950's sparse matrix cores:
//
//   D = alpha * A * op(B) + beta * C,   A: m x k with at most 2 nonzeros in every group of 4
//                                        consecutive k, given compressed (values + indices)
//
// Sparse tensor cores as the page "稀疏张量核心加速模板计算的技术解析" (sparse tensor cores for stencil
// computation) describes them in sections 1.2.1 and 1.3.2: a 2:4 sparse
// operand is held as its kept values (half of k) plus 2 bits of metadata per kept value (its
// position within its group of 4), and the matrix instruction skips the zeros.  Here the
// instruction is v_smfmac_f32_16x16x64_{f16,bf16}: a 16 x 16 output block over 64 logical k
// from A's kept values (lane group g: the 8 kept values of k 16 g .. 16 g + 15, 16 bytes),
// B's 64 k-rows (two 32-k fragments of the dense layout, 32 bytes) and a 16-bit index (2 bits
// per kept value, low half of the register) -- lane layouts measured on gfx950.
//
// The pipeline is the dense kernel's (mpgemm_kernel.hpp): direct-to-LDS loads of each stage
// into one of two LDS buffers, fragments of the next k step read during the current one, one
// barrier per stage.  A stage is 128 logical k: A's 64 kept values per row (128 bytes, the
// dense K-contiguous operand geometry), B's 128 k-rows as two dense stages of 64, and the
// metadata's 16 bytes per row (one 1 KB load per wave).  The tile is 256 x 128 (LDS 136 KB);
// k must be a multiple of 128 (no K tail), m and n are arbitrary.
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

typedef __attribute__((address_space(3))) unsigned short lds_u16;

}  // namespace

template <int IN, int OUT, bool TB>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void sp24_kernel(SpParams sp) {
    const Params &p = sp.p;
    constexpr int BM = kSpTileM, BN = kSpTileN;
    constexpr int FM = BM / 32, FN = BN / 32;       // 16-wide blocks per wave (2 x 2 waves)
    using OpA = Operand<2, true, BM / 32>;          // kept values: K-contiguous, 64 per stage
    using OpB = Operand<2, TB, BN / 32>;            // each 64-k-row half of a stage of B
    constexpr int A_BYTES = OpA::kStageBytes;       // 32 KB
    constexpr int BH_BYTES = OpB::kStageBytes;      // 16 KB
    constexpr int B_BYTES = 2 * BH_BYTES;
    constexpr int M_BYTES = BM * 16;                // metadata: 16 bytes per row per stage
    constexpr int B_BASE = kBuffers * A_BYTES, M_BASE = B_BASE + kBuffers * B_BYTES;
    constexpr int kLoads = OpA::kSlots + 2 * OpB::kSlots + 1;   // per wave per stage

    // LDS: [A0 | A1 | B0 (k-rows 0-63, 64-127) | B1 | M0 | M1]
    __shared__ __attribute__((aligned(16))) char smem_raw[M_BASE + kBuffers * M_BYTES];
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
    OpB opb_lo, opb_hi;
    opa.init(wave, lane, p.lda, m_left, 0u);
    opb_lo.init(wave, lane, p.ldb, n_left, (uint32_t)B_BASE);
    opb_hi.init(wave, lane, p.ldb, n_left, (uint32_t)(B_BASE + BH_BYTES));
    const int nk = p.k / 128;                        // stages (k is a multiple of 128)

    // Stage cursors (see StageCursor): the exact readable end of each operand bounds the
    // last stage.  A's rows hold k / 2 kept values; B's two halves are 64 k-rows apart.
    StageCursor ca, cb_lo, cb_hi, cm;
    {
        const int64_t kc = p.k / 2;
        const int64_t end_a = (int64_t)(p.m - 1) * p.lda * 2 + ((kc * 2 + 15) & ~(int64_t)15);
        const int64_t rb = TB ? p.n : p.k, clb = TB ? p.k : p.n;
        const int64_t end_b = (rb - 1) * p.ldb * 2 + ((clb * 2 + 15) & ~(int64_t)15);
        const int64_t end_m = (int64_t)(p.m - 1) * sp.ld_meta + (((int64_t)p.k / 8 + 15) & ~(int64_t)15);
        const int64_t off_a = (int64_t)m0 * p.lda * 2;
        const int64_t off_b = TB ? (int64_t)n0 * p.ldb * 2 : (int64_t)n0 * 2;
        const int64_t half_b = TB ? 128 : (int64_t)64 * p.ldb * 2;   // k-rows 64..127 of a stage
        const int64_t off_m = (int64_t)m0 * sp.ld_meta;
        ca.step = kStageKBytes;
        cb_lo.step = cb_hi.step = TB ? 256 : (int64_t)128 * p.ldb * 2;
        cm.step = 16;
        ca.base = (uint64_t)p.A + (uint64_t)off_a;
        cb_lo.base = (uint64_t)p.B + (uint64_t)off_b;
        cb_hi.base = cb_lo.base + (uint64_t)half_b;
        cm.base = (uint64_t)sp.meta + (uint64_t)off_m;
        auto last = [&](int64_t end, int64_t off, int64_t step) {
            const int64_t l = end - off - (int64_t)(nk > 0 ? nk - 1 : 0) * step;
            return (int)(l < 0 ? 0 : (l > kNumRecords ? kNumRecords : l));
        };
        ca.last_records = last(end_a, off_a, ca.step);
        cb_lo.last_records = last(end_b, off_b, cb_lo.step);
        cb_hi.last_records = last(end_b, off_b + half_b, cb_hi.step);
        cm.last_records = last(end_m, off_m, cm.step);
    }
    // metadata load: lane l of wave w brings row 64 w + l (clamped to the last row)
    const uint32_t voff_m = (uint32_t)min(64 * wave + lane, m_left - 1) * (uint32_t)sp.ld_meta;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};

    const uint32_t lds_w = (uint32_t)(uintptr_t)smem + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
    i32x4 rs_a, rs_lo, rs_hi, rs_m;
    auto next_rsrc = [&](int s) {
        rs_a = ca.rsrc(s, nk);
        ca.advance();
        rs_lo = cb_lo.rsrc(s, nk);
        cb_lo.advance();
        rs_hi = cb_hi.rsrc(s, nk);
        cb_hi.advance();
        rs_m = cm.rsrc(s, nk);
        cm.advance();
    };
    auto load_slot = [&](int parity, int l) {
        if (l < OpA::kSlots) {
            opa.load(rs_a, lds_w + (uint32_t)(parity * A_BYTES), l);
        } else if (l < OpA::kSlots + OpB::kSlots) {
            opb_lo.load(rs_lo, lds_w + (uint32_t)(B_BASE + parity * B_BYTES), l - OpA::kSlots);
        } else if (l < kLoads - 1) {
            opb_hi.load(rs_hi, lds_w + (uint32_t)(B_BASE + parity * B_BYTES + BH_BYTES),
                        l - OpA::kSlots - OpB::kSlots);
        } else {
            dma16(rs_m, voff_m, 0u, lds_w + (uint32_t)(M_BASE + parity * M_BYTES));
        }
    };

    // Fragments of one k step (64 logical k): A's kept values, B's two 32-k fragments, the
    // index.  Two sets: the next k step's are read during the current one.
    u32x4 fa[2][FM];
    u32x8 fb[2][FN];
    uint32_t fi[2][FM];
    // metadata of row (16 i + lane % 16) of this wave's rows, k step t, lane group g
    const uint32_t m_lane = (uint32_t)((wm * (BM / 2) + lane % 16) * 16 + 2 * (lane / 16));
    constexpr int kUnits = FM + 2 * FN + FM, kMf = FM * FN;
    auto read_unit = [&](int set, int parity, int t, int u) {
        if (u < FM) {
            fa[set][u] = opa.frag(smem + parity * A_BYTES, wm * FM + u, t);
        } else if (u < FM + 2 * FN) {
            const int j = (u - FM) / 2, h = (u - FM) % 2;
            const lds_char *st = smem + parity * B_BYTES;
            set_half(fb[set][j], h, t == 0 ? opb_lo.frag(st, wn * FN + j, h) : opb_hi.frag(st, wn * FN + j, h));
        } else {
            const int i = u - FM - 2 * FN;
            fi[set][i] = *(const lds_u16 *)(smem + M_BASE + parity * M_BYTES + m_lane + i * 256 + 8 * t);
        }
    };

    // One k step: FM x FN sparse MFMAs of fragment set `set`, each in its own fenced group
    // with at most a few other instructions; the next k step's fragments are read spread over
    // the MFMAs; in the second k step of a stage the loads of the stage two ahead.
    auto k_step = [&](auto set_c, int rd_parity, int rd_t, int ld_parity, auto nl_c, auto &&hook) {
        constexpr int set = decltype(set_c)::value, nl = decltype(nl_c)::value;
        wait_lds<0>();
        static_for<kMf>([&](auto idx_c) {
            constexpr int idx = decltype(idx_c)::value;
            constexpr int i = idx / FN, j = idx % FN;
            SMma<IN>::run(fa[set][i], fb[set][j], fi[set][i], acc[i][j]);
            hook(idx_c);
            static_for<kUnits>([&](auto u_c) {
                constexpr int u = decltype(u_c)::value;
                constexpr int at = (u * kMf) / kUnits;
                if constexpr (at == idx) read_unit(set ^ 1, rd_parity, rd_t, u);
            });
            static_for<nl>([&](auto l_c) {
                constexpr int l = decltype(l_c)::value;
                constexpr int at = ((l * kMf) / (nl > 0 ? nl : 1) + 1) % kMf;
                if constexpr (at == idx) load_slot(ld_parity, l);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using CL = std::integral_constant<int, kLoads>;
    auto stage_iter = [&](int s, auto par_c) {
        constexpr int P = decltype(par_c)::value;
        k_step(C0{}, P, 1, 0, C0{}, [&](auto idx_c) {
            if constexpr (decltype(idx_c)::value == 1 % kMf) next_rsrc(s + 2);
        });
        wait_vmem<0>();  // this wave's loads of stage s + 1 have landed
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        k_step(C1{}, P ^ 1, 0, P, CL{}, [&](auto) {});
    };

    // Prologue: stages 0 and 1 queued, stage 0 waited for, the first k step's fragments read.
    next_rsrc(0);
    static_for<kLoads>([&](auto l_c) { load_slot(0, decltype(l_c)::value); });
    next_rsrc(1);
    static_for<kLoads>([&](auto l_c) { load_slot(1, decltype(l_c)::value); });
    wait_vmem<kLoads>();
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnits; ++u) read_unit(0, 0, 0, u);
    for (int s = 0; s < nk; s += 2) {
        stage_iter(s, C0{});
        stage_iter(s + 1, C1{});
    }
    wait_vmem<0>();  // no direct load into LDS is left in flight when the workgroup ends
    drain_mfma(acc);
    store_tile<false, OUT, FM, FN, BM, BN>(p, acc, m0, n0, wm, wn, lane, full_mn, m_left, n_left);
}

template __global__ void sp24_kernel<IN_F16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, true>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, true>(SpParams);

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
    return hipErrorInvalidValue;
}

}  // namespace mpg
