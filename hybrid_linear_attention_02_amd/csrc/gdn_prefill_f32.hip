// Prefill of float32 inputs: the chunked gated delta rule on the fp32 MFMA
// (v_mfma_f32_16x16x4_f32), for results within fp32 rounding of the token
// recurrence.
//
// The chunk form is the one of the bf16 prefill (the WY / UT form of the
// delta rule over chunks of C = 64 tokens):
//
//   U  = T diag(beta) (V - diag(exp(gamma) rk) K H)
//   O  = diag(exp(gamma) rq) Q H + P U
//   H' = exp(gamma_last) H + K^T diag(rk exp(gamma_last - gamma)) U
//
// with raw q and k rows, their L2 norms applied as the row scales rk and rq
// (rq includes the attention scale). The intra-chunk kernel of the bf16
// prefill, instantiated for float32 rows, computes T = (I + A)^-1, P and the
// per-token scale rows of every (chunk, value head) into the workspace, with
// every product on the fp32 MFMA. This file holds the recurrence across
// chunks.
//
// Recurrence: one workgroup of four waves per (sequence, value head, 16
// value columns); the columns of H evolve independently under the rule, so a
// single long sequence still spreads over dv / 16 workgroups per head. Per
// chunk, wave w owns the 16-token row block w for the products over tokens
// and the dk blocks t = w, w + 4, ... of the fp32 master state, which it keeps
// in accumulators:
//   X_w = K_w H and Z_w = Q_w H               (B operand: H, transposed in LDS)
//   R_w = beta (V_w - exp(gamma) rk X_w)      -> LDS, barrier
//   U_w = sum_{j <= w} T_wj R_j               -> LDS, barrier
//   O_w = exp(gamma) rq Z_w + sum_{j <= w} P_wj U_j
//   H'_t = exp(gamma_last) H_t + sum_j K_j^T (D U)_j   -> LDS, barrier
// X, Z and O are formed one row per lane (the accumulator layout of their
// transposes), so v is loaded and o stored with one 16-byte access per lane.
// The chunk's K tile (read transposed by the state advance), its T and P
// blocks and its scale rows are staged in double-buffered LDS, each wave
// loading a share; the wave's own q rows and v go straight to registers.
// Everything is loaded one chunk ahead, the loads interleaved with the
// products: a CU's vector memory unit takes load instructions one at a time,
// and issued as one block they held the waves for a third of a chunk.
// Workgroups of one (sequence, head) are placed on one XCD so that they share
// its L2 for q, k, T and P.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gdn_internal.h"
#include "gdn_prefill_common.h"

namespace {

using namespace gdn::pf;

template <int DK>
struct F32Tiles {
    static_assert(DK % 16 == 0 && DK >= 16 && DK <= 128, "dk must be 16, 32, 64 or 128");
    static constexpr int SK = DK + 4;        // LDS row stride (floats) of the K tile and of H^T
    static constexpr int NB = DK / 16;       // 16-row blocks of dk
    static constexpr int NT = (NB + 3) / 4;  // state blocks per wave (block t belongs to wave t % 4)
    static constexpr int KV = DK / 16;       // float4s of the 64 x DK K tile per thread
};

// Operands of one chunk as loaded from global memory (one chunk ahead).
// Token rows are held "one row per lane": lane (row, g) = (lane % 16, lane / 16)
// holds 4 consecutive columns 4 g .. 4 g + 3 of its row.
template <int DK>
struct F32Chunk {
    f32x4 kst[F32Tiles<DK>::KV];  // K tile: float4 number tid + 256 u (row-major, DK / 4 per row) -> LDS
    f32x4 qa[F32Tiles<DK>::NB];   // Q[16 w + row][16 b + 4 g ..]: this wave's rows, block b of dk
    f32x4 v;                      // V[16 w + row][c0 + 4 g ..]
    f32x4 tp[5];                  // fragments 5 w .. 5 w + 4 of the chunk's 20 T and P blocks -> LDS
    f32x4 sc;                     // float4 number 64 w + lane of the 80 of the scale rows -> LDS
    int ck;                       // checkpoint slot after the chunk (< 0: none)
};

// First chunk of sequence n (kernel-argument table for small calls, indexed
// by constants only so it stays in the argument segment).
__device__ __forceinline__ int chunk_base(const PrefillParams& p, int n) {
    if (p.inl_n > 0) {
        int r = 0;
#pragma unroll
        for (int i = 0; i < kInlineSeqs; ++i)
            if (i == n) r = p.inl_chunk[i];
        return r;
    }
    return p.chunk_off[n];
}

constexpr int kTP = 20;                    // T and P blocks of a (chunk, head) in the workspace
constexpr int kScF4 = kScRows * kC / 4;    // float4s of its scale rows
constexpr int kSR = kC + 4;                // LDS row stride (floats) of R, stored column-major

template <int DK>
__global__ void __launch_bounds__(256) prefill_f32_recurrent_kernel(PrefillParams p, int ncg, int npairs) {
    using S = F32Tiles<DK>;
    constexpr int SK = S::SK, NB = S::NB, NT = S::NT, KV = S::KV;
    // chunk operands shared by the waves, double-buffered (chunk i in buffer i % 2)
    __shared__ __align__(16) float sK[2][64 * SK];       // K tile, row-major
    __shared__ __align__(16) f32x4 sTP[2][kTP][64];      // T blocks 0..9, then P blocks, as fragments
    __shared__ __align__(16) float sSc[2][kScRows * kC]; // scale rows
    __shared__ __align__(16) float sH[16 * SK];          // H^T: sH[col * SK + dk row]
    __shared__ __align__(16) float sR[16 * kSR];         // R^T: sR[col * kSR + token]
    __shared__ __align__(16) f32x4 sU[4][64];            // U_w in accumulator layout

    // blocks are dealt to the 8 XCDs round-robin: the ncg column groups of
    // one (sequence, head) pair get block numbers that agree mod 8
    const unsigned blk = blockIdx.x;
    const int slot8 = static_cast<int>(blk >> 3);
    const int pair = (slot8 / ncg) * 8 + static_cast<int>(blk & 7);
    if (pair >= npairs) return;
    const int n = pair / p.hv, h = pair - n * p.hv;
    const int c0 = (slot8 % ncg) * 16;
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: its branches stay scalar
    const int dv = p.dv;

    const int d = p.dst[n];
    if (d < 0) return;                                // sequence skipped
    const int s = p.src[n];
    const int j = h / p.group;
    const int t0 = p.cu[n], t1 = p.cu[n + 1];
    const int nch = (t1 - t0 + kC - 1) / kC;
    const int cb = chunk_base(p, n);
    // (token and chunk ranges as the host mirror of cu_seqlens promised)
    if (d >= p.num_slots || s >= p.num_slots || t1 > p.total_tokens || t1 < t0 || cb + nch > p.num_chunks) {
        if (tid == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
        return;
    }
    const size_t tile = static_cast<size_t>(DK) * dv;

    // fp32 master state: blocks t = w + 4 u of H (dk rows 16 t ..), lane
    // (col, g) holding H[16 t + 4 g + e][c0 + col]
    f32x4 hm[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int t = w + 4 * u;
        hm[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < NB && s >= 0) {
            const float* in = p.pool + (static_cast<size_t>(s) * p.hv + h) * tile + c0 + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) hm[u][e] = in[static_cast<size_t>(16 * t + 4 * g4 + e) * dv];
        }
    }
    const auto store_state = [&](int slot) {
        float* out = p.pool + (static_cast<size_t>(slot) * p.hv + h) * tile + c0 + l16;
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const int t = w + 4 * u;
            if (t < NB)
#pragma unroll
                for (int e = 0; e < 4; ++e) out[static_cast<size_t>(16 * t + 4 * g4 + e) * dv] = hm[u][e];
        }
    };
    const auto put_state_lds = [&]() {
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const int t = w + 4 * u;
            if (t < NB) *reinterpret_cast<f32x4*>(sH + l16 * SK + 16 * t + 4 * g4) = hm[u];
        }
    };

    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    // Token rows through buffer resources spanning the chunk's valid rows:
    // rows past the sequence end read as zero and are not stored, so no load
    // or store needs a branch (and every wave issues the same loads, which
    // keeps the wait counts exact).
    const unsigned kq_row = static_cast<unsigned>(p.hk) * DK;     // floats between token rows of q and k
    const unsigned v_row = static_cast<unsigned>(p.hv) * dv;      // ... of v and o
    const auto kq_rsrc = [&](const float* x, int r0, int len) {
        return make_rsrc(x + (static_cast<size_t>(r0) * p.hk + j) * DK, 4u * ((len - 1) * kq_row + DK));
    };
    const auto vo_rsrc = [&](const float* x, int r0, int len) {
        return make_rsrc(x + (static_cast<size_t>(r0) * p.hv + h) * dv + c0, 4u * ((len - 1) * v_row + 16));
    };
    // Loads of chunk i's operands, in three parts that the chunk before it
    // spreads over its products: a CU's vector memory unit takes each load
    // instruction in turn, and issued all at once they would hold the waves
    // for most of a chunk.
    struct Rsrc {
        rsrc_t k, q;
    };
    const auto chunk_rows = [&](int i) {
        const int r0 = t0 + kC * i;
        return Rsrc{kq_rsrc(p.kf, r0, min(kC, t1 - r0)), kq_rsrc(p.qf, r0, min(kC, t1 - r0))};
    };
    const auto fetch_kq = [&](const Rsrc& r, F32Chunk<DK>& in, int b) {   // K tile part b, Q rows block b
        const unsigned q4 = tid + 256 * b, row = q4 / (DK / 4), col4 = q4 % (DK / 4);
        in.kst[b] = buf_load_f4(r.k, 4u * (row * kq_row + 4 * col4));
        in.qa[b] = buf_load_f4(r.q, 4u * ((16 * w + l16) * kq_row + 16 * b + 4 * g4));
    };
    const auto fetch_tp = [&](int i, F32Chunk<DK>& in) {
        const size_t mat = (static_cast<size_t>(cb + i) * p.hv + h) * 2;   // T, then P (contiguous)
        const f32x4* tpr = reinterpret_cast<const f32x4*>(p.tpf + mat * kFragFloats) + (5 * w) * 64 + lane;
#pragma unroll
        for (int u = 0; u < 5; ++u) in.tp[u] = tpr[u * 64];
    };
    const auto fetch_rest = [&](int i, F32Chunk<DK>& in) {
        const int r0 = t0 + kC * i;
        in.v = buf_load_f4(vo_rsrc(p.vf, r0, min(kC, t1 - r0)), 4u * ((16 * w + l16) * v_row + 4 * g4));
        const rsrc_t scr = make_rsrc(p.sc + (static_cast<size_t>(cb + i) * p.hv + h) * (kScRows * kC), 16u * kScF4);
        in.sc = buf_load_f4(scr, 16u * (64 * w + lane));
        in.ck = p.ckpt != nullptr ? p.ckpt[cb + i] : -1;
    };
    const auto stage_k = [&](const F32Chunk<DK>& in, int buf, int u) {
        const int q4 = tid + 256 * u, row = q4 / (DK / 4), col4 = q4 - row * (DK / 4);
        *reinterpret_cast<f32x4*>(sK[buf] + row * SK + 4 * col4) = in.kst[u];
    };
    const auto stage_tp_sc = [&](const F32Chunk<DK>& in, int buf) {
#pragma unroll
        for (int u = 0; u < 5; ++u) sTP[buf][5 * w + u][lane] = in.tp[u];
        if (64 * w + lane < kScF4) *reinterpret_cast<f32x4*>(sSc[buf] + 4 * (64 * w + lane)) = in.sc;
    };

    // One chunk; `nxt` receives the operands of chunk i + 1 meanwhile (the
    // last chunk loads and stages its own operands again: unconditional
    // loads keep the wait counts exact, so using `cur` never waits for them).
    const auto chunk = [&](int i, const F32Chunk<DK>& cur, F32Chunk<DK>& nxt) {
        const int inext = i + 1 < nch ? i + 1 : i;
        const Rsrc rn = chunk_rows(inext);
        const int buf = i & 1;
        const float* kt = sK[buf];
        const float* sc = sSc[buf];
        const int r0 = t0 + kC * i;
        const int len = min(kC, t1 - r0);
        const int tr = 16 * w + l16;                  // this lane's token row (row-per-lane layouts)
        const int f0 = w * (w + 1) / 2;               // first T block of row block w

        // Every LDS operand that is ready is read in bulk ahead of the
        // products (the scheduler would otherwise sink each read to its use
        // and expose the LDS latency once per block).
        f32x4 hb[NB], ka[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            hb[b] = *reinterpret_cast<const f32x4*>(sH + l16 * SK + 16 * b + 4 * g4);
            ka[b] = *reinterpret_cast<const f32x4*>(kt + tr * SK + 16 * b + 4 * g4);
        }
        // K rows as columns for the state advance: kc[u][jb][e] =
        // K[16 jb + 4 g + e][16 t + col], t = w + 4 u
        f32x4 kc[NT][4];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const int t = w + 4 * u;
            if (t < NB) {
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) kc[u][jb][e] = kt[(16 * jb + 4 * g4 + e) * SK + 16 * t + l16];
            }
        }
        // blocks (w, jb) of T and P, zero above the diagonal
        f32x4 tf[4], pf[4], scd[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const f32x4 tv = sTP[buf][f0 + (jb <= w ? jb : w)][lane];
            const f32x4 pv = sTP[buf][10 + f0 + (jb <= w ? jb : w)][lane];
            tf[jb] = jb <= w ? tv : zero;
            pf[jb] = jb <= w ? pv : zero;
            scd[jb] = *reinterpret_cast<const f32x4*>(sc + kScD * kC + 16 * jb + 4 * g4);
        }
        const float scx = sc[kScX * kC + tr], bet = sc[kScBeta * kC + tr], scz = sc[kScZ * kC + tr];
        const float sce = sc[kScE * kC];
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products

        // X_w = K_w H and Z_w = Q_w H, one row per lane (the accumulator
        // layout of (K_w H)^T), contraction k = 16 b + 4 g + e; the next
        // chunk's K tile and q rows are requested block by block in between
        f32x4 x = zero, z = zero;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            x = mm16(hb[b], ka[b], x);
            z = mm16(hb[b], cur.qa[b], z);
            fetch_kq(rn, nxt, b);
            __builtin_amdgcn_sched_barrier(0);
        }
        // R_w = beta (V_w - exp(gamma) rk X_w), stored transposed
        const f32x4 rw = bet * (cur.v - scx * x);
#pragma unroll
        for (int e = 0; e < 4; ++e) sR[(4 * g4 + e) * kSR + tr] = rw[e];
        lds_barrier();

        // U_w = sum_{jb <= w} T_w,jb R_jb (accumulator layout)
        f32x4 rr[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) rr[jb] = *reinterpret_cast<const f32x4*>(sR + l16 * kSR + 16 * jb + 4 * g4);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 uw = zero;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) uw = mm16(tf[jb], rr[jb], uw);
        sU[w][lane] = uw;
        lds_barrier();

        // H'_t = exp(gamma_last) H_t + sum_jb (K_jb rows as columns) (D U)_jb,
        // interleaved with O_w = exp(gamma) rq Z_w + sum_jb P_w,jb U_jb (one
        // row per lane: the accumulator layout of (P U)^T); in between, the
        // next chunk's K tile goes to LDS and its T, P, v and scale rows are
        // requested
        f32x4 uu[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) uu[jb] = sU[jb][lane];
        __builtin_amdgcn_sched_barrier(0);
        f32x4 ou = scz * z;
        f32x4 acc[NT];
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[u] = sce * hm[u];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const f32x4 du = scd[jb] * uu[jb];
#pragma unroll
            for (int u = 0; u < NT; ++u)
                if (w + 4 * u < NB) acc[u] = mm16(kc[u][jb], du, acc[u]);
            ou = mm16(uu[jb], pf[jb], ou);
#pragma unroll
            for (int u = jb; u < KV; u += 4) stage_k(nxt, buf ^ 1, u);
            if (jb == 0) fetch_tp(inext, nxt);
            if (jb == 2) fetch_rest(inext, nxt);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = 0; u < NT; ++u)
            if (w + 4 * u < NB) hm[u] = acc[u];
        buf_store16(__builtin_bit_cast(u32x4, ou), vo_rsrc(p.of, r0, len), 4u * (tr * v_row + 4 * g4));
        put_state_lds();
        {
            const int slot = __builtin_amdgcn_readfirstlane(cur.ck);
            if (slot >= p.num_slots) {
                if (tid == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
            } else if (slot >= 0) {
                store_state(slot);
            }
        }
        stage_tp_sc(nxt, buf ^ 1);
        lds_barrier();
    };

    if (nch > 0) {
        F32Chunk<DK> ring[2];
        {
            const Rsrc r = chunk_rows(0);
#pragma unroll
            for (int b = 0; b < NB; ++b) fetch_kq(r, ring[0], b);
            fetch_tp(0, ring[0]);
            fetch_rest(0, ring[0]);
#pragma unroll
            for (int u = 0; u < KV; ++u) stage_k(ring[0], 0, u);
            stage_tp_sc(ring[0], 0);
        }
        put_state_lds();
        lds_barrier();
        int i = 0;
        for (; i + 2 <= nch; i += 2) {
            chunk(i, ring[0], ring[1]);
            chunk(i + 1, ring[1], ring[0]);
        }
        if (i < nch) chunk(i, ring[0], ring[1]);
    }
    store_state(d);
}

template <int DK>
int launch_rec(const PrefillParams& p, hipStream_t s) {
    const int ncg = p.dv / 16;
    const int npairs = p.n_seqs * p.hv;
    const dim3 grid(static_cast<unsigned>(8 * ncg * ((npairs + 7) / 8)));
    hipLaunchKernelGGL((prefill_f32_recurrent_kernel<DK>), grid, dim3(256), 0, s, p, ncg, npairs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked: fp32 recurrence launch failed: ") +
                                        hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

namespace gdn {
namespace pf {

int launch_f32_recurrence(const PrefillParams& p, hipStream_t s) {
    switch (p.dkq) {
        case 16: return launch_rec<16>(p, s);
        case 32: return launch_rec<32>(p, s);
        case 64: return launch_rec<64>(p, s);
        case 128: return launch_rec<128>(p, s);
        default: return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: unsupported dk");
    }
}

}  // namespace pf
}  // namespace gdn
