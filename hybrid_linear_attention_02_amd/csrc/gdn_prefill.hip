// Chunked prefill of the gated delta rule over a slot pool (gfx950).
//
// Every sequence (packed by cu_seqlens) is cut into chunks of C = 64 tokens,
// restarting at each sequence boundary. Inside a chunk of c tokens, with
// cumulative log-decay gamma_r = sum_{s<=r} g_s, k^/q~ the normalised keys and
// scaled queries, and H the dk x dv state at the chunk start (H = S^T), the
// token recurrence is exactly
//
//   A[r,s] = beta_r exp(gamma_r - gamma_s) (k^_r . k^_s)   (s < r)
//   T      = (I + A)^-1                                    (unit lower triangular)
//   U      = T diag(beta) (V - diag(exp(gamma)) K^ H)      (the per-token updates u_r)
//   P[r,s] = exp(gamma_r - gamma_s) (q~_r . k^_s)          (s <= r)
//   O      = diag(exp(gamma)) Q~ H + P U
//   H'     = exp(gamma_last) H + K^T diag(exp(gamma_last - gamma)) U
//
// (the WY / UT form of the delta rule, applied as T times one bracket). Decay
// factors are always exp of a non-positive difference.
//
// Kernels, after a tiny chunk-offset prep:
//  * intra-chunk, one wave per (chunk, value head), all chunks in parallel:
//    the raw q / k rows of the chunk are held in registers in MFMA operand
//    layout, row norms and the Gram matrices K K^T and Q K^T come from them
//    on 16x16x32 bf16 MFMA, A goes to LDS (column-major), and T is solved in
//    fp32 by a right-looking substitution (lane = column of T; each step
//    broadcasts one column of A and updates every later row, so the serial
//    chain is one FMA per row). T, P and five per-token scale rows go to the
//    workspace.
//  * recurrence, one workgroup per (sequence, value head, 16*NW value
//    columns), sequential over the chunks of its sequence. The fp32 master
//    state lives in MFMA accumulators; X = K H, Z = Q H, U = T Y,
//    O = diag(.) Z + P U and H' = e H + K^T (D U) are bf16 MFMA contractions.
//    K^T and V are read transposed straight from the row-major LDS tiles with
//    the gfx950 LDS transpose read, so no transposed copy is ever stored. The
//    next chunk's operands are fetched into registers while the current chunk
//    is computed (one LDS buffer, two barriers per chunk), and the output tile
//    is staged in LDS and written with 16-byte stores.
//
// Raw (unnormalised) bf16 q and k are the MFMA operands; the L2 norms and the
// decay factors are applied as fp32 row scales on the accumulator side.
//
// float32 inputs use the same intra-chunk kernel instantiated for fp32 rows
// (Gram products on the fp32 MFMA, T and P written as fp32 blocks) and the
// fp32 recurrence of gdn_prefill_f32.hip; the parameter block, the sequence
// lookup and the small helpers both files share are in
// gdn_prefill_common.h.

#include <hip/hip_runtime.h>
#include <type_traits>

#include <cstdint>
#include <string>

#include "gdn_internal.h"
#include "gdn_prefill_common.h"

namespace {

using namespace gdn::pf;

// Uniform base pointer plus a 32-bit per-lane byte offset: lets the compiler
// use the scalar-base global access form (no 64-bit address per lane).
template <typename T, typename B>
__device__ __forceinline__ T* at_bytes(B* base, unsigned byte_off) {
    using C = typename std::conditional<std::is_const<B>::value, const char, char>::type;
    return reinterpret_cast<T*>(reinterpret_cast<C*>(base) + byte_off);
}
template <typename T, typename B>
__device__ __forceinline__ const T* at_bytes(const B* base, unsigned byte_off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Byte range of `rows` token rows of `width` bf16 values, rows `stride`
// elements apart (zero rows: an empty range).
__device__ __forceinline__ unsigned rows_bytes(int rows, unsigned stride, int width) {
    return rows > 0 ? 2u * ((rows - 1) * stride + width) : 0u;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// float -> bfloat16, round to nearest even, on the gfx950 packed convert
// (v_cvt_pk_bf16_f32); NaN stays NaN.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }


// 8 bf16 from two fp32 accumulator quads: slots 0-3 <- a, 4-7 <- b.
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
    u32x4 w;
    w.x = pack_bf16x2(a.x, a.y);
    w.y = pack_bf16x2(a.z, a.w);
    w.z = pack_bf16x2(b.x, b.y);
    w.w = pack_bf16x2(b.z, b.w);
    return as_bf16x8(w);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// K-slot convention shared by every operand below: inside a 32-wide k block,
// slot e (e < 4) of lane group g = lane / 16 is k = 4g + e and slot 4 + e is
// k = 16 + 4g + e. An fp32 accumulator pair (rows base..base+15 and
// base+16..base+31, lane = column, 4 rows 4g..4g+3 per lane) packed with
// pack8 has exactly this order, so results feed the next contraction
// directly.

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane j receives element (j & 3) of the 4 consecutive 16-bit values loaded
// by lanes 4e + (j >> 2), for e = 0..3. Pointing lane i of group g at
// M[row0 + 4g + (i >> 2)][col0 + 4 (i & 3)] therefore hands lane (g, j) the
// column values M[row0 + 4g + e][col0 + j], e = 0..3.
__device__ __forceinline__ i16x4 lds_tr4_raw(const uint16_t* buf, int stride, int row0, int col0, int g4, int l16) {
    const uint16_t* a = buf + (row0 + 4 * g4 + (l16 >> 2)) * stride + col0 + 4 * (l16 & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
}

// M[row0 + 4g + e][col0 + lane % 16] for e = 0..3 as fp32: a column slice in
// accumulator layout.
__device__ __forceinline__ f32x4 lds_tr4_f32(const uint16_t* buf, int stride, int row0, int col0, int g4, int l16) {
    const i16x4 r = lds_tr4_raw(buf, stride, row0, col0, g4, l16);
    f32x4 out;
    out.x = bf16_to_f32(static_cast<uint16_t>(r.x));
    out.y = bf16_to_f32(static_cast<uint16_t>(r.y));
    out.z = bf16_to_f32(static_cast<uint16_t>(r.z));
    out.w = bf16_to_f32(static_cast<uint16_t>(r.w));
    return out;
}

// LDS bank model behind the layouts below (measured on gfx950 with the
// SQ_LDS_BANK_CONFLICT counter): 64 banks of 4 bytes; a single 8-byte-per-lane
// read is served 32 lanes per pass and is conflict-free when those lanes'
// 64 dwords sit in distinct banks. When the compiler fuses two such reads
// into one two-address instruction, that instruction costs extra cycles even
// if each half alone would be conflict-free; so every layout below also makes
// the address difference between any two operand reads depend on the lane,
// which the compiler cannot fuse.
//
// Tiles are stored with unpadded rows of G 8-byte granules, and granule j of
// row r sits at granule j ^ swz(r), where swz(r) is even (16-byte pairs stay
// aligned and contiguous, so 16-byte staging writes are unchanged) and is the
// XOR of a per-row term and a per-16-row-group constant that also differs
// between tiles of the same shape.

// q/k tiles (64 rows x DK bf16), read as MFMA row operands (16 rows x 2
// granules per pass) and through the transpose read (8 consecutive rows x 4
// consecutive granules per pass). Per-row term 4 ((r >> a) & m) +
// 2 ((r >> 3) & 1), with a = log2(32 / G) and m = G / 4 - 1: the 16 rows of a
// row-operand read get 16 distinct granule offsets (2 ... 32 / G rows share
// one pass of banks), the 8 rows of a transpose read differ above the
// 4-granule span. Group constant 2 (r >> 4), plus 8 for the q tile.
template <int DK, bool IS_Q>
__device__ __forceinline__ int kq_swz(int r) {
    constexpr int G = DK / 4;
    constexpr int A = (G == 32) ? 0 : (G == 16) ? 1 : 2;
    constexpr int M = G / 4 - 1;
    static_assert(G == 8 || G == 16 || G == 32, "dk must be 32, 64 or 128");
    const int group = (2 * (r >> 4) + (IS_Q ? 8 : 0)) & (G - 2);
    return (4 * ((r >> A) & M) + 2 * ((r >> 3) & 1)) ^ group;
}

// element offset of (row r, column col) in a swizzled q/k tile; col % 4 == 0
template <int DK, bool IS_Q>
__device__ __forceinline__ int kq_off(int r, int col) {
    return r * DK + 4 * ((col >> 2) ^ kq_swz<DK, IS_Q>(r)) + (col & 3);
}

// Row operand from a swizzled q/k tile: slots = M[row][base + k(slot)].
template <int DK, bool IS_Q>
__device__ __forceinline__ bf16x8 kq_pair(const uint16_t* buf, int row, int base, int g4) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(buf + kq_off<DK, IS_Q>(row, base + 4 * g4));
    const u32x2 hi = *reinterpret_cast<const u32x2*>(buf + kq_off<DK, IS_Q>(row, base + 16 + 4 * g4));
    u32x4 w;
    w.x = lo.x;
    w.y = lo.y;
    w.z = hi.x;
    w.w = hi.y;
    return as_bf16x8(w);
}

// Transposed operand from a swizzled k tile: slots = M[row0 + k(slot)][col0 + lane % 16].
template <int DK>
__device__ __forceinline__ bf16x8 kq_tr_pair(const uint16_t* buf, int row0, int col0, int g4, int l16) {
    const int r = row0 + 4 * g4 + (l16 >> 2);
    const int c = col0 + 4 * (l16 & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + kq_off<DK, false>(r, c)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + kq_off<DK, false>(r + 16, c)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    u32x4 w;
    w.x = l2.x;
    w.y = l2.y;
    w.z = h2.x;
    w.w = h2.y;
    return as_bf16x8(w);
}


// ---------------------------------------------------------------------------
// prep: first chunk and first segment of every sequence
// ---------------------------------------------------------------------------

// Exclusive prefix sums of the chunk and segment counts of every sequence,
// 1024 sequences per round: a scan inside each wave, then the wave totals
// through LDS. (A zero-length sequence has no chunk but one segment, which
// carries its state to the destination.)
constexpr int kOffThreads = 1024;

__global__ void __launch_bounds__(kOffThreads) chunk_offsets_kernel(PrefillParams p) {
    constexpr int NWV = kOffThreads / 64;
    __shared__ int32_t wc[NWV], ws[NWV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int32_t carry_c = 0, carry_s = 0;
    for (int base = 0; base < p.n_seqs; base += kOffThreads) {
        const int i = base + tid;
        int32_t nc = 0, ns = 0;
        if (i < p.n_seqs) {
            const int32_t len = p.cu[i + 1] - p.cu[i];
            nc = len > 0 ? (len + kC - 1) / kC : 0;
            ns = (p.seg_len == 0 || nc <= p.seg_len) ? 1 : (nc + p.seg_len - 1) / p.seg_len;
        }
        int32_t xc = nc, xs = ns;               // inclusive scan inside the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t yc = __shfl_up(xc, off), ys = __shfl_up(xs, off);
            if (lane >= off) {
                xc += yc;
                xs += ys;
            }
        }
        if (lane == 63) {
            wc[w] = xc;
            ws[w] = xs;
        }
        __syncthreads();
        int32_t oc = carry_c, os = carry_s, tc = 0, ts = 0;
#pragma unroll
        for (int k = 0; k < NWV; ++k) {
            if (k < w) {
                oc += wc[k];
                os += ws[k];
            }
            tc += wc[k];
            ts += ws[k];
        }
        if (i < p.n_seqs) {
            p.chunk_off_w[i] = oc + xc - nc;
            p.seg_off_w[i] = os + xs - ns;
        }
        carry_c += tc;
        carry_s += ts;
        __syncthreads();                        // wc / ws are rewritten next round
    }
    if (tid == 0) {
        p.chunk_off_w[p.n_seqs] = carry_c;
        p.seg_off_w[p.n_seqs] = carry_s;
    }
}


// ---------------------------------------------------------------------------
// intra-chunk: one wave per (chunk, key head), for every value head of the
// key head's group
// ---------------------------------------------------------------------------

// F32: float32 q and k (any dk that is a multiple of 16), Gram matrices on the
// fp32 MFMA, T and P written as fp32 row fragments (p.tpf); otherwise bf16
// q and k, Gram matrices on the bf16 MFMA, T and P as bf16 row-operand
// fragments (p.tp). The decay, A, the solve for T and the scale rows are the
// same fp32 arithmetic in both.
template <int DK, bool F32>
__global__ void __launch_bounds__(64) prefill_intra_kernel(PrefillParams p) {
    constexpr int KS = F32 ? 1 : DK / 32;   // bf16 MFMA k-steps over dk
    // The four 16 x 16 diagonal blocks of a 64 x 64 matrix in LDS: block b
    // at b * BS floats, rows of 16 floats. The 16-float gap between blocks
    // puts the four lane groups (one per block) on different banks.
    constexpr int SD = 16;            // row stride (floats)
    constexpr int BS = 16 * SD + 16;  // block stride (floats)
    // diagonal blocks of A (row-major) until the solve has read them, then
    // of T (column-major): the workgroup is one wave, so every read of A
    // precedes the first write of T
    __shared__ __align__(16) float sAT[4 * BS];
    __shared__ __align__(16) float sTr[4 * BS];        // diagonal blocks of T, row-major
    __shared__ __align__(16) float sGam[kC], sBeta[kC], sRk[kC], sRq[kC];

    const int c = blockIdx.x;
    const int j = blockIdx.y;                // key head
    const int lane = threadIdx.x & 63;       // one wave: lets the compiler bound g4 below
    const int g4 = lane >> 4, l16 = lane & 15;
    if (c >= p.num_chunks) return;
    const SeqSpan sp = find_span<false>(p, c);
    const int n = sp.n;
    const int t0 = p.cu[n] + (c - sp.c0) * kC;
    const int tend = p.cu[n + 1];
    const int len = min(kC, tend - t0);
    if (len <= 0 || tend > p.total_tokens || p.dst[n] < 0) return;

    // per-token g, beta of value head h (token = lane)
    const auto load_gb = [&](int h, float& gl, float& bl) {
        gl = 0.f;
        bl = 0.f;
        if (lane < len) {
            const size_t gi = static_cast<size_t>(t0 + lane) * p.hv + h;
            gl = p.g[gi];
            bl = p.beta[gi];
        }
    };
    float gl_next, bl_next;
    // Shared by the group's value heads: the L2 norms of the k and q rows
    // (row scales rk in sRk, rq = scale / |q| in rqv and sRq) and the raw Gram
    // tiles with one row per lane (each product takes the column tile's k
    // rows as its first operand): gkk[tr][ts] = K_ts K_tr^T, gkq = K_ts Q_tr^T,
    // ts <= tr, packed as index tr (tr + 1) / 2 + ts.
    float rqv[4];
    f32x4 gkk[10], gkq[10];
    if constexpr (F32) {
        load_gb(j * p.group, gl_next, bl_next);
        // fp32 rows in blocks of 16 features, lane (row, g) holding
        // X[row][16 b + 4 g + e]; sums of squares and the Gram tiles
        // accumulate block by block
        float sk[4] = {0.f, 0.f, 0.f, 0.f}, sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 10; ++i) {
            gkk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            gkq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // Rows through buffer resources over the chunk's valid rows (rows past
        // the end read as zero), one block of 16 features in flight ahead of
        // the products on the current one; the loop is kept rolled so the
        // wave needs few enough registers for two waves per SIMD.
        const unsigned kq_row = static_cast<unsigned>(p.hk) * DK;
        const unsigned kq_bytes = 4u * ((len - 1) * kq_row + DK);
        const rsrc_t kr = make_rsrc(p.kf + (static_cast<size_t>(t0) * p.hk + j) * DK, kq_bytes);
        const rsrc_t qr = make_rsrc(p.qf + (static_cast<size_t>(t0) * p.hk + j) * DK, kq_bytes);
        const auto load_block = [&](int b, f32x4* kx, f32x4* qx) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const unsigned off = 4u * ((16 * tt + l16) * kq_row + 16 * b + 4 * g4);
                kx[tt] = buf_load_f4(kr, off);
                qx[tt] = buf_load_f4(qr, off);
            }
        };
        f32x4 kb[4], qb[4];
        load_block(0, kb, qb);
#pragma unroll 1
        for (int b = 0; b < DK / 16; ++b) {
            f32x4 kn[4], qn[4];
            load_block(b + 1 < DK / 16 ? b + 1 : b, kn, qn);   // (the last block loads itself again)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sk[tt] += kb[tt][e] * kb[tt][e];
                    sq[tt] += qb[tt][e] * qb[tt][e];
                }
#pragma unroll
            for (int tr = 0; tr < 4; ++tr)
#pragma unroll
                for (int ts = 0; ts <= tr; ++ts) {
                    const int ix = tr * (tr + 1) / 2 + ts;
                    gkk[ix] = mm16(kb[ts], kb[tr], gkk[ix]);
                    gkq[ix] = mm16(kb[ts], qb[tr], gkq[ix]);
                }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                kb[tt] = kn[tt];
                qb[tt] = qn[tt];
            }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            float a = sk[tt], b = sq[tt];
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            b += __shfl_xor(b, 16);
            b += __shfl_xor(b, 32);
            const int r = 16 * tt + l16;
            rqv[tt] = (r < len) ? p.scale * __builtin_amdgcn_rsqf(b + p.eps) : 0.f;
            if (g4 == 0) {
                sRk[r] = (r < len) ? __builtin_amdgcn_rsqf(a + p.eps) : 0.f;
                sRq[r] = rqv[tt];
            }
        }
    } else {
        // raw k and q rows as row operands in natural feature order (a
        // contraction over dk may order its k slots freely, as long as both
        // operands agree): kr[tt][ks] = K[16 tt + l16][32 ks + 8 g .. +7]. All
        // of them are requested before any is used, so the wave waits for one
        // global round trip, not five.
        const auto load_rows = [&](const uint16_t* x, int tt, u32x4* dst) {
            const int r = 16 * tt + l16;
            const size_t base = (static_cast<size_t>(t0 + r) * p.hk + j) * p.dkq + 8 * g4;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                dst[ks] = (r < len && 32 * ks + 8 * g4 < p.dkq) ? *reinterpret_cast<const u32x4*>(x + base + 32 * ks)
                                                                 : u32x4{0u, 0u, 0u, 0u};
        };
        // sum of squares of the row held in operand layout, over all four lane groups
        const auto row_sumsq = [&](const u32x4* xr) {
            float acc = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = __uint_as_float(xr[ks][e] << 16), x1 = __uint_as_float(xr[ks][e] & 0xffff0000u);
                    acc += x0 * x0 + x1 * x1;
                }
            acc += __shfl_xor(acc, 16);
            acc += __shfl_xor(acc, 32);
            return acc;
        };
        u32x4 kr[4][KS], qa[4][KS];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) load_rows(p.k, tt, kr[tt]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) load_rows(p.q, tt, qa[tt]);
        load_gb(j * p.group, gl_next, bl_next);

        // norms from fp32 sums of the exact bf16 squares, Gram tiles on the
        // bf16 MFMA
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float sk = row_sumsq(kr[tt]);
            const int r = 16 * tt + l16;
            if (g4 == 0) sRk[r] = (r < len) ? __builtin_amdgcn_rsqf(sk + p.eps) : 0.f;
        }
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int r = 16 * tr + l16;
            rqv[tr] = (r < len) ? p.scale * __builtin_amdgcn_rsqf(row_sumsq(qa[tr]) + p.eps) : 0.f;
            if (g4 == 0) sRq[r] = rqv[tr];
        }
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int ts = 0; ts <= tr; ++ts) {
                f32x4 kk = f32x4{0.f, 0.f, 0.f, 0.f}, kq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 bk = as_bf16x8(kr[ts][ks]);
                    kk = mfma16(bk, as_bf16x8(kr[tr][ks]), kk);
                    kq = mfma16(bk, as_bf16x8(qa[tr][ks]), kq);
                }
                gkk[tr * (tr + 1) / 2 + ts] = kk;
                gkq[tr * (tr + 1) / 2 + ts] = kq;
            }
    }

    for (int hig = 0; hig < p.group; ++hig) {
        const int h = j * p.group + hig;
        const float gl = gl_next, bl = bl_next;
        if (hig + 1 < p.group) load_gb(h + 1, gl_next, bl_next);
        // cumulative log-decay by an inclusive lane scan, in base 2
        // (gamma log2(e)), so every decay factor is one hardware exp2
        float gam = gl * 1.4426950408889634f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_up(gam, off);
            if (lane >= off) gam += t;
        }
        const float gam_last = __shfl(gam, 63);   // padded tokens add g = 0
        lds_barrier();                          // the previous head's LDS reads are done
        sGam[lane] = gam;
        sBeta[lane] = bl;
        lds_barrier();

        // A (strictly lower), kept in registers off the diagonal and in LDS
        // on it, and P, which goes to the workspace as row-operand fragments
        const size_t mat = (static_cast<size_t>(c) * p.hv + h) * 2;     // T of this (chunk, head); P follows
        u32x4* Pf = F32 ? nullptr : reinterpret_cast<u32x4*>(p.tp + (mat + 1) * (kC * kC));
        f32x4* Pf32 = F32 ? reinterpret_cast<f32x4*>(p.tpf + (mat + 1) * kFragFloats) : nullptr;
        f32x4 ra[6];                           // A blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int r = 16 * tr + l16;       // this lane's row
            const float rq = rqv[tr];
            const float gr = sGam[r], brk = sBeta[r] * sRk[r];
            f32x4 pt[4];                       // pt[ts][e] = P[r][16 ts + 4 g + e]
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                pt[ts] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (ts > tr) continue;
                const f32x4 kk = gkk[tr * (tr + 1) / 2 + ts], kq = gkq[tr * (tr + 1) / 2 + ts];
                const f32x4 gs = *reinterpret_cast<const f32x4*>(sGam + 16 * ts + 4 * g4);
                const f32x4 rks = *reinterpret_cast<const f32x4*>(sRk + 16 * ts + 4 * g4);
                f32x4 a;
                // below the diagonal block every column precedes the row (the
                // masks fold away there); gr - gs <= 0 wherever the mask keeps it
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sc = 16 * ts + 4 * g4 + e;
                    float dec = exp2_hw(gr - gs[e]);
                    if (ts == tr) dec = (sc <= r) ? dec : 0.f;
                    const float dr = dec * rks[e];
                    a[e] = (ts < tr || sc < r) ? brk * dr * kk[e] : 0.f;
                    pt[ts][e] = rq * dr * kq[e];
                }
                if (ts == tr) *reinterpret_cast<f32x4*>(sAT + tr * BS + l16 * SD + 4 * g4) = a;
                else ra[tr * (tr - 1) / 2 + ts] = a;
            }
            if constexpr (F32) {
#pragma unroll
                for (int ts = 0; ts <= tr; ++ts) Pf32[(tr * (tr + 1) / 2 + ts) * 64 + lane] = pt[ts];
            } else {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)   // (rows below 32 have an all-zero second k-step: not written)
                    if (ks == 0 || tr >= 2)
                        Pf[(tr * 2 + ks) * 64 + lane] = __builtin_bit_cast(u32x4, pack8(pt[2 * ks], pt[2 * ks + 1]));
            }
        }
        lds_barrier();
        {
            const float rk = sRk[lane], rq = sRq[lane];
            const float eg = exp2_hw(gam);
            float* scp = p.sc + (static_cast<size_t>(c) * p.hv + h) * (kScRows * kC);
            scp[kScX * kC + lane] = eg * rk;
            scp[kScBeta * kC + lane] = bl;
            scp[kScZ * kC + lane] = eg * rq;
            scp[kScD * kC + lane] = rk * exp2_hw(gam_last - gam);
            scp[kScE * kC + lane] = exp2_hw(gam_last);
        }

        // T = (I + A)^-1, blocked by 16. The four diagonal blocks
        // T_bb = (I + A_bb)^-1 are solved at once, lane group b taking block b,
        // lane t of it column t, by forward substitution over the block's rows.
        {
            const int bb = g4, t = l16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float* arow = sAT + bb * BS + r * SD;
                float acc = (r == t) ? 1.f : 0.f;
#pragma unroll
                for (int s4 = 0; s4 < r; s4 += 4) {
                    const f32x4 av = *reinterpret_cast<const f32x4*>(arow + s4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (s4 + e < r) acc -= av[e] * x[s4 + e];
                }
                x[r] = acc;
            }
#pragma unroll
            for (int r4 = 0; r4 < 16; r4 += 4)
                *reinterpret_cast<f32x4*>(sAT + bb * BS + t * SD + r4) = f32x4{x[r4], x[r4 + 1], x[r4 + 2], x[r4 + 3]};
#pragma unroll
            for (int r = 0; r < 16; ++r) sTr[bb * BS + r * SD + t] = x[r];
        }
        lds_barrier();
        // diagonal blocks in both operand layouts: C (lane = column) and R (lane = row)
        f32x4 tc[3], trf[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            if (bb < 3) tc[bb] = *reinterpret_cast<const f32x4*>(sAT + bb * BS + l16 * SD + 4 * g4);
            trf[bb] = *reinterpret_cast<const f32x4*>(sTr + bb * BS + l16 * SD + 4 * g4);
        }
        // Off the diagonal, T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj), level by
        // level on the fp32 MFMA; blocks used again later are kept in layout C,
        // every block is produced in layout R for the output.
        const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 S;
        S = mm16(ra[0], tc[0], z);                                    // A10 T00
        const f32x4 t10c = -mm16(trf[1], S, z), t10r = -mm16(S, trf[1], z);
        S = mm16(ra[2], tc[1], z);                                    // A21 T11
        const f32x4 t21c = -mm16(trf[2], S, z), t21r = -mm16(S, trf[2], z);
        S = mm16(ra[5], tc[2], z);                                    // A32 T22
        const f32x4 t32r = -mm16(S, trf[3], z);
        S = mm16(ra[2], t10c, mm16(ra[1], tc[0], z));                 // A20 T00 + A21 T10
        const f32x4 t20c = -mm16(trf[2], S, z), t20r = -mm16(S, trf[2], z);
        S = mm16(ra[5], t21c, mm16(ra[4], tc[1], z));                 // A31 T11 + A32 T21
        const f32x4 t31r = -mm16(S, trf[3], z);
        S = mm16(ra[5], t20c, mm16(ra[4], t10c, mm16(ra[3], tc[0], z)));   // A30 T00 + A31 T10 + A32 T20
        const f32x4 t30r = -mm16(S, trf[3], z);

        if constexpr (F32) {
            // T to the workspace as fp32 row fragments of its ten lower blocks
            f32x4* Tf = reinterpret_cast<f32x4*>(p.tpf + mat * kFragFloats);
            auto put = [&](int tau, int jb, f32x4 x) { Tf[(tau * (tau + 1) / 2 + jb) * 64 + lane] = x; };
            put(0, 0, trf[0]);
            put(1, 0, t10r);
            put(1, 1, trf[1]);
            put(2, 0, t20r);
            put(2, 1, t21r);
            put(2, 2, trf[2]);
            put(3, 0, t30r);
            put(3, 1, t31r);
            put(3, 2, t32r);
            put(3, 3, trf[3]);
        } else {
            // T to the workspace as row-operand fragments (tau, ks) = rows 16 tau ..,
            // k block 32 ks: blocks (tau, 2 ks) and (tau, 2 ks + 1); the two all-zero
            // fragments (0, 1) and (1, 1) are not written
            u32x4* Tf = reinterpret_cast<u32x4*>(p.tp + mat * (kC * kC));
            auto put = [&](int tau, int ks, f32x4 lo, f32x4 hi) {
                Tf[(tau * 2 + ks) * 64 + lane] = __builtin_bit_cast(u32x4, pack8(lo, hi));
            };
            put(0, 0, trf[0], z);
            put(1, 0, t10r, trf[1]);
            put(2, 0, t20r, t21r);
            put(2, 1, trf[2], z);
            put(3, 0, t30r, t31r);
            put(3, 1, t32r, trf[3]);
        }
    }
}

// ---------------------------------------------------------------------------
// recurrence: one workgroup per (segment, value head, NV = 16 NW value columns)
//
// Two wave roles, one of each per SIMD:
//   compute waves (NW, one per 16 value columns) run only the state chain of
//     each chunk, X = K H, Y, U = T Y, H' = e H + K^T D U, from
//     double-buffered LDS tiles; in output mode they also publish H (bf16, as
//     used for X) and U (bf16) of the chunk;
//   helper waves (4, one per 16-token row block of a chunk) stage the next
//     chunk's K, T, V and scale rows into the other LDS buffer and, one step
//     behind, form the outputs O = diag(exp(gamma) rq) Q H + P U of their rows
//     from q and P rows they load straight into registers and the published
//     H and U.
// A step is one chunk for the compute waves; every wave meets one workgroup
// barrier per step. The state chain, the critical path of a sequence, thus
// carries no global memory traffic, staging or output work.
// ---------------------------------------------------------------------------

template <int DK, int NW, int MODE>
struct RecShape {
    static constexpr bool OUT = MODE == 0;
    static constexpr int NV = 16 * NW;        // value columns per workgroup
    static constexpr int NA = 64 * NW;        // compute threads (waves 0 .. NW-1)
    static constexpr int NB = 256;            // helper threads (waves NW .. NW+3)
    static constexpr int NT = NA + NB;
    static constexpr int KS = DK / 32;        // k-steps over dk
    static constexpr int MT = DK / 16;        // 16-row tiles of the state
    static constexpr int SV = NV + 16;        // bf16 row stride of the V slice
    static constexpr int SO = NV + 8;         // bf16 row stride of a helper's output tile
    static constexpr int KP = 8 * DK;         // 16-byte pieces: K tile
    static constexpr int TPP = 512;           //                 T tile
    static constexpr int VP = 8 * NV;         //                 V slice
    static constexpr int SCP = kScRows * kC / 4;   //            scale rows
    static constexpr int KQ = (KP + NB - 1) / NB;  // per helper thread
    static constexpr int TP = TPP / NB;
    static constexpr int VV = (VP + NB - 1) / NB;
    static constexpr int SCN = (SCP + NB - 1) / NB;
    // LDS layout in bytes; the two buffers of each tile are adjacent so that
    // one address register serves both (the second through the immediate).
    static constexpr int SZ_K = kC * DK * 2, SZ_T = kC * kC * 2, SZ_V = kC * SV * 2, SZ_SC = kScRows * kC * 4;
    static constexpr int SZ_H = NV * DK * 2, SZ_U = NV * kC * 2;
    static constexpr int L_K = 0;
    static constexpr int L_T = L_K + 2 * SZ_K;
    static constexpr int L_V = L_T + 2 * SZ_T;
    static constexpr int L_SC = L_V + 2 * SZ_V;
    static constexpr int L_H = L_SC + 2 * SZ_SC;
    static constexpr int L_U = L_H + (OUT ? 2 * SZ_H : 0);
    static constexpr int L_O = L_U + (OUT ? 2 * SZ_U : 0);
    static constexpr int BYTES = L_O + (OUT ? 4 * 16 * SO * 2 : 0);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(TP * NB == TPP, "tile split");
};

// Column-major bf16 tiles exchanged between the two roles (H: NV columns of
// DK features in natural order, 16-byte piece j = features 8 j .. 8 j + 7;
// U: NV columns of 64 tokens, piece j = tokens 32 (j / 4) + {4 (j % 4) + e,
// 16 + 4 (j % 4) + e}, the operand slot order). Piece j of column n sits at
// piece j ^ f(n). Rows of 16 R bytes pack 16 / R columns into one 256-byte
// bank line; f(n) = (n / (16 / R)) mod R then gives the 16 columns of a pass
// 16 distinct 16-byte bank groups.
template <int R>
__device__ __forceinline__ int cm_off(int n, int j) {
    constexpr int PER = 16 / R;
    return n * (16 * R) + 16 * (j ^ ((n / PER) & (R - 1)));
}

// Work unit of the recurrence: one segment of one sequence (a whole sequence
// when the prefill is not split).
struct Segment {
    int n;          // sequence
    int c0, c1;     // chunk range [c0, c1)
    int tb, te;     // token range [tb, te)
    bool first, last;
    bool split;     // the sequence has more than one segment
    int k;          // index of the segment in its sequence
    int g0;         // first segment of the sequence
};

__device__ __forceinline__ Segment locate_segment(const PrefillParams& p, int g) {
    Segment sg;
    const SeqSpan sp = find_span<true>(p, g);
    sg.n = sp.n;
    const int k = g - sp.s0;
    const int nseg = sp.s1 - sp.s0;
    const int cs = sp.c0, ce = sp.c1;
    sg.k = k;
    sg.g0 = sp.s0;
    sg.first = k == 0;
    sg.last = k == nseg - 1;
    sg.split = nseg > 1;
    sg.c0 = nseg == 1 ? cs : cs + k * p.seg_len;
    sg.c1 = sg.last ? ce : sg.c0 + p.seg_len;
    sg.tb = p.cu[sg.n] + (sg.c0 - cs) * kC;
    sg.te = sg.last ? p.cu[sg.n + 1] : sg.tb + (sg.c1 - sg.c0) * kC;
    return sg;
}

// Modes of the recurrence kernel.
enum : int {
    kModeOutput = 0,   // outputs o, state from the slot / zero / segment initial state, final state to the slot
    kModeState = 1,    // split pass 1: no outputs; columns [0, dv) carry the state from zero with V,
                       // columns [dv, dv + dk) carry the identity with V = 0 (the transition M);
                       // results to the segment buffers. The first segment instead carries the
                       // true initial state (no transition), so its result is the next start; the
                       // output pass carries later segments' starts through the transitions.
};

// Registers a helper wave loads one step ahead for its output rows.
template <int KS>
struct HelperRows {
    bf16x8 q[KS];     // q rows as row operands
    bf16x8 pr[2];     // P rows as row operands (k-steps over the 64 tokens)
    f32x4 sz;         // exp(gamma) rq of its 4 rows
};

template <int DK, int NW, int MODE>
__global__ void __launch_bounds__(64 * NW + 256)
prefill_recurrent_kernel(PrefillParams p) {
    using S = RecShape<DK, NW, MODE>;
    constexpr bool OUT = S::OUT;
    constexpr int NV = S::NV, NA = S::NA, KS = S::KS, MT = S::MT;
    constexpr int SV = S::SV, SO = S::SO;
    constexpr int KQ = S::KQ, TP = S::TP, VV = S::VV, SCN = S::SCN;
    __shared__ __align__(16) unsigned char lds[S::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g4 = lane >> 4, l16 = lane & 15;
    const bool helper = tid >= NA;
    // index within the role, in a scalar register (wave-uniform addresses
    // and buffer resources derived from it stay scalar)
    const int wave = __builtin_amdgcn_readfirstlane((helper ? tid - NA : tid) >> 6);
    // blockIdx.x -> (key head, value head in its group, column group), key
    // head fastest so that the workgroups sharing one key head's q/k rows sit
    // on the same XCD (workgroups are dealt to the 8 XCDs round robin).
    const int j = blockIdx.x % p.hk;
    const int rest = blockIdx.x / p.hk;
    const int hig = rest % p.group;
    const int grp = rest / p.group;
    const int h = j * p.group + hig;
    const Segment sg = locate_segment(p, blockIdx.y);
    const int n = sg.n;
    if (!OUT && sg.last) return;              // the last segment's end state is not needed

    const int dsl = p.dst[n];
    if (dsl < 0) return;
    const int ssl = p.src[n];
    const int tb = sg.tb, te = sg.te;
    const int c0 = sg.c0, c1 = sg.c1;
    if (dsl >= p.num_slots || ssl >= p.num_slots || te > p.total_tokens || te < tb || c1 > p.num_chunks) {
        if (tid == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
        return;
    }
    // columns of this workgroup: value columns [vcol0, vcol0 + NV); in the
    // state pass, groups past dv carry columns of the transition instead
    const int ncg = p.dv / NV;
    const bool m_cols = !OUT && grp >= ncg;
    // The first segment of a split sequence starts from the true initial
    // state (source slot or zero), so its end state needs no transition.
    if (m_cols && sg.first) return;
    const int vcol0 = (m_cols ? grp - ncg : grp) * NV;
    const int nch = c1 - c0;

    auto tile16 = [&](int off, int b, int size) {
        return reinterpret_cast<uint16_t*>(lds + off + b * size);
    };

    // ---------------- helper role: staging ----------------
    // Every helper step issues the same loads and stores with no branch
    // around them (the counts of outstanding memory operations then stay
    // exact, so a wait covers only what it needs): chunk indices are clamped
    // into the segment, and rows past a chunk's end or a disabled store fall
    // outside a buffer resource's range, where loads return zero and stores
    // are dropped.
    const unsigned kq_row = static_cast<unsigned>(p.hk) * p.dkq;   // elements between token rows
    const unsigned v_row = static_cast<unsigned>(p.hv) * p.dv;
    const int htid = tid - NA;
    constexpr unsigned kOff = 0x80000000u;      // offset past every range
    u32x4 rK[KQ], rT[TP], rV[VV], rS[SCN];
    auto chunk_len = [&](int c) { return min(kC, te - (tb + (c - c0) * kC)); };
    auto fetch = [&](int c) {
        const int t0 = tb + (c - c0) * kC;
        const int len = chunk_len(c);
        const rsrc_t kr = make_rsrc(p.k + (static_cast<size_t>(t0) * p.hk + j) * p.dkq, rows_bytes(len, kq_row, p.dkq));
#pragma unroll
        for (int m = 0; m < KQ; ++m) {
            const int idx = htid + S::NB * m;
            const int r = idx / (DK / 8), c8 = idx % (DK / 8);
            rK[m] = buf_load16(kr, 8 * c8 < p.dkq ? 2u * (r * kq_row + c8 * 8) : kOff);   // padded columns: zero
        }
        // T fragments; the two all-zero ones, (0, 1) and (1, 1), are never
        // written by the intra-chunk kernel nor read here (they load as zero)
        const rsrc_t tr_ = make_rsrc(p.tp + (static_cast<size_t>(c) * p.hv + h) * 2 * (kC * kC), 2u * (kC * kC));
#pragma unroll
        for (int m = 0; m < TP; ++m) {
            const int idx = htid + S::NB * m, frag = idx >> 6;
            rT[m] = buf_load16(tr_, (frag == 1 || frag == 3) ? kOff : 16u * idx);
        }
        const rsrc_t vr = make_rsrc(p.v + (static_cast<size_t>(t0) * p.hv + h) * p.dv + vcol0,
                                    m_cols ? 0u : rows_bytes(len, v_row, NV));
#pragma unroll
        for (int m = 0; m < VV; ++m) {
            const int idx = htid + S::NB * m;
            const int r = idx / (NV / 8), c8 = idx % (NV / 8);
            rV[m] = buf_load16(vr, idx < S::VP ? 2u * (r * v_row + 8 * c8) : kOff);
        }
        const rsrc_t sr = make_rsrc(p.sc + (static_cast<size_t>(c) * p.hv + h) * (kScRows * kC), 16u * S::SCP);
#pragma unroll
        for (int m = 0; m < SCN; ++m) {
            const int idx = htid + S::NB * m;
            rS[m] = buf_load16(sr, idx < S::SCP ? 16u * idx : kOff);
        }
    };
    auto stage = [&](int b) {
        uint16_t* sK = tile16(S::L_K, b, S::SZ_K);
        uint16_t* sT = tile16(S::L_T, b, S::SZ_T);
        uint16_t* sV = tile16(S::L_V, b, S::SZ_V);
        float* sSc = reinterpret_cast<float*>(lds + S::L_SC + b * S::SZ_SC);
#pragma unroll
        for (int m = 0; m < KQ; ++m) {
            const int idx = htid + S::NB * m;
            const int r = idx / (DK / 8), c8 = idx % (DK / 8);
            *reinterpret_cast<u32x4*>(sK + kq_off<DK, false>(r, c8 * 8)) = rK[m];
        }
#pragma unroll
        for (int m = 0; m < TP; ++m) *reinterpret_cast<u32x4*>(sT + 8 * (htid + S::NB * m)) = rT[m];
        // (transition columns stage the zeros their empty buffer range loads)
#pragma unroll
        for (int m = 0; m < VV; ++m) {
            const int idx = htid + S::NB * m;
            const int r = idx / (NV / 8), c8 = idx % (NV / 8);
            if (idx < S::VP) *reinterpret_cast<u32x4*>(sV + r * SV + c8 * 8) = rV[m];
        }
#pragma unroll
        for (int m = 0; m < SCN; ++m) {
            const int idx = htid + S::NB * m;
            if (idx < S::SCP) *reinterpret_cast<u32x4*>(sSc + 4 * idx) = rS[m];
        }
    };

    // ---------------- helper role: outputs ----------------
    // helper wave w owns chunk rows [16 w, 16 w + 16)
    // q rows as row operands in natural feature order (lane (g, row) takes
    // features 32 ks + 8 g .. +7, matching the published H); P rows come as
    // row-operand fragments written by the intra-chunk kernel, one contiguous
    // kilobyte per (row tile, k-step)
    auto fetch_rows = [&](int c, HelperRows<KS>& hr) {
        const int t0 = tb + (c - c0) * kC;
        const rsrc_t qr = make_rsrc(p.q + (static_cast<size_t>(t0) * p.hk + j) * p.dkq, rows_bytes(chunk_len(c), kq_row, p.dkq));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            hr.q[ks] = __builtin_bit_cast(bf16x8, buf_load16(qr, 32 * ks + 8 * g4 < p.dkq
                                                                     ? 2u * ((16 * wave + l16) * kq_row + 32 * ks + 8 * g4)
                                                                     : kOff));
        // (the second k-step of P is all zero for rows below 32 and is then not used)
        const rsrc_t pr_ = make_rsrc(p.tp + (static_cast<size_t>(c) * p.hv + h) * 2 * (kC * kC) + kC * kC, 2u * (kC * kC));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            hr.pr[ks] = __builtin_bit_cast(bf16x8, buf_load16(pr_, (ks == 1 && wave < 2) ? kOff : 16u * ((wave * 2 + ks) * 64 + lane)));
        const float* SCg = p.sc + (static_cast<size_t>(c) * p.hv + h) * (kScRows * kC);
        hr.sz = *at_bytes<f32x4>(SCg, 4u * (kScZ * kC + 16 * wave + 4 * g4));
    };
    // outputs of the helper's rows of a chunk from buffer b, as bf16 row
    // pieces in registers
    constexpr int OP = 16 * NV / 8;               // 16-byte pieces in the wave's 16 x NV tile
    constexpr int OPL = (OP + 63) / 64;           // per lane
    auto emit_rows = [&](int b, const HelperRows<KS>& hr, u32x4 (&ov)[OPL]) {
        const unsigned char* sH = lds + S::L_H + b * S::SZ_H;
        const unsigned char* sU = lds + S::L_U + b * S::SZ_U;
        f32x4 acc[NW];
#pragma unroll
        for (int ct = 0; ct < NW; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Z = Q H (contraction over dk), H read back column-major: lane
        // (g, column) takes features 32 ks + 8 g .. +7, as its q fragment
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 hbv[NW];
#pragma unroll
            for (int ct = 0; ct < NW; ++ct)
                hbv[ct] = *reinterpret_cast<const bf16x8*>(sH + cm_off<DK / 8>(16 * ct + l16, 4 * ks + g4));
#pragma unroll
            for (int ct = 0; ct < NW; ++ct) acc[ct] = mfma16(hr.q[ks], hbv[ct], acc[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < NW; ++ct) acc[ct] *= hr.sz;
        // + P U (contraction over the chunk's tokens)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks == 1 && wave < 2) break;
            bf16x8 ubv[NW];
#pragma unroll
            for (int ct = 0; ct < NW; ++ct)
                ubv[ct] = *reinterpret_cast<const bf16x8*>(sU + cm_off<8>(16 * ct + l16, 4 * ks + g4));
#pragma unroll
            for (int ct = 0; ct < NW; ++ct) acc[ct] = mfma16(hr.pr[ks], ubv[ct], acc[ct]);
        }
        // through the wave's own LDS tile to 16-byte row stores
        uint16_t* sO = reinterpret_cast<uint16_t*>(lds + S::L_O) + wave * 16 * SO;
#pragma unroll
        for (int ct = 0; ct < NW; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) sO[(4 * g4 + i) * SO + 16 * ct + l16] = f32_to_bf16(acc[ct][i]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
        for (int m = 0; m < OPL; ++m) {
            const int idx = lane + 64 * m;
            const int r = idx / (NV / 8), c8 = idx % (NV / 8);
            ov[m] = *reinterpret_cast<const u32x4*>(sO + (idx < OP ? r * SO + c8 * 8 : 0));
        }
    };
    // store the rows emitted for chunk c (last in a helper step: no wait of
    // the step then queues behind the stores); nothing is stored when `live`
    // is false
    auto store_rows = [&](int c, bool live, const u32x4 (&ov)[OPL]) {
        const int t0 = tb + (c - c0) * kC;
        const int len = chunk_len(c) - 16 * wave;   // rows of this wave's block inside the chunk
        const rsrc_t orr = make_rsrc(p.o + (static_cast<size_t>(t0 + 16 * wave) * p.hv + h) * p.dv + vcol0,
                                     live ? rows_bytes(len, v_row, NV) : 0u);
#pragma unroll
        for (int m = 0; m < OPL; ++m) {
            const int idx = lane + 64 * m;
            const int r = idx / (NV / 8), c8 = idx % (NV / 8);
            buf_store16(ov[m], orr, idx < OP ? 2u * (r * v_row + 8 * c8) : kOff);
        }
    };

    // ---------------- compute role ----------------
    const int col = vcol0 + wave * 16 + l16;    // this lane's column (value or transition)
    // fp32 master state: H[mu][i] = H[16 mu + 4 g + i][col]
    f32x4 H[MT];
    if (!helper) {
        const float* init = nullptr;
        int init_rows = DK;                     // rows of the source tile (pool tiles have dkq)
        if (OUT) {
            // A split sequence starts its first segment from the state pass's
            // copy of the initial state (the source slot is then read only by
            // that pass, before the last segment may overwrite it in place),
            // its second from the first segment's end state, and later ones
            // from that state carried through the transitions below.
            if (sg.split) {
                init = (sg.k == 0 ? p.sh : p.se) + (static_cast<size_t>(sg.g0) * p.hv + h) * (static_cast<size_t>(DK) * p.dv);
            } else if (ssl >= 0) {
                init = p.pool + (static_cast<size_t>(ssl) * p.hv + h) * (static_cast<size_t>(p.dkq) * p.dv);
                init_rows = p.dkq;
            }
        } else if (sg.first && ssl >= 0) {
            init = p.pool + (static_cast<size_t>(ssl) * p.hv + h) * (static_cast<size_t>(p.dkq) * p.dv);
            init_rows = p.dkq;
        }
        if (init != nullptr) {
#pragma unroll
            for (int mu = 0; mu < MT; ++mu)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * mu + 4 * g4 + i;
                    H[mu][i] = row < init_rows ? init[row * p.dv + col] : 0.f;
                }
        } else {
#pragma unroll
            for (int mu = 0; mu < MT; ++mu)
#pragma unroll
                for (int i = 0; i < 4; ++i) H[mu][i] = (m_cols && 16 * mu + 4 * g4 + i == col) ? 1.f : 0.f;
        }
    }
    auto chunk = [&](int b) {
        const uint16_t* sK = tile16(S::L_K, b, S::SZ_K);
        const uint16_t* sT = tile16(S::L_T, b, S::SZ_T);
        const uint16_t* sV = tile16(S::L_V, b, S::SZ_V);
        const float* sSc = reinterpret_cast<const float*>(lds + S::L_SC + b * S::SZ_SC);
        // state pass: the operands of Y, U and DU (scale rows, V, the T
        // fragments) do not depend on the state, so they are requested before
        // the X products (the output pass has no registers to spare for them)
        f32x4 ysx[4], ysb[4], yv[4], ysd[4];
        bf16x8 ytf[6];
        if (!OUT) {
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const int r0 = 16 * tau + 4 * g4;
                ysx[tau] = *reinterpret_cast<const f32x4*>(sSc + kScX * kC + r0);
                ysb[tau] = *reinterpret_cast<const f32x4*>(sSc + kScBeta * kC + r0);
                yv[tau] = lds_tr4_f32(sV, SV, 16 * tau, wave * 16, g4, l16);
            }
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int tau = i < 4 ? i : i - 2, ks = i < 4 ? 0 : 1;
                ytf[i] = *reinterpret_cast<const bf16x8*>(sT + 8 * ((tau * 2 + ks) * 64 + lane));
            }
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) ysd[tau] = *reinterpret_cast<const f32x4*>(sSc + kScD * kC + 16 * tau + 4 * g4);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 hb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) hb[ks] = pack8(H[2 * ks], H[2 * ks + 1]);
        // X = K H (contraction over dk); k-step outer so that each step's
        // operand reads overlap the previous step's MFMAs
        f32x4 X[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) X[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 ak[4];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) ak[tau] = kq_pair<DK, false>(sK, 16 * tau + l16, 32 * ks, g4);
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) X[tau] = mfma16(ak[tau], hb[ks], X[tau]);
        }
        if (OUT) {
            // publish the chunk's initial state for the helpers' Q H, column
            // by column in natural feature order (the helpers' q fragments
            // hold 8 consecutive features per lane): rows 16 mu + 4 g .. +3
            // are the half (g & 1) of 16-byte piece 2 mu + (g >> 1)
            unsigned char* sH = lds + S::L_H + b * S::SZ_H;
            const int n = 16 * wave + l16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 w = __builtin_bit_cast(u32x4, hb[ks]);
                *reinterpret_cast<u32x2*>(sH + cm_off<DK / 8>(n, 4 * ks + (g4 >> 1)) + 8 * (g4 & 1)) = u32x2{w.x, w.y};
                *reinterpret_cast<u32x2*>(sH + cm_off<DK / 8>(n, 4 * ks + 2 + (g4 >> 1)) + 8 * (g4 & 1)) = u32x2{w.z, w.w};
            }
        }
        // Y = diag(beta) (V - diag(exp(gamma) rk) X)
        f32x4 Y[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            if (!OUT) {
                Y[tau] = ysb[tau] * (yv[tau] - ysx[tau] * X[tau]);
            } else {
                const int r0 = 16 * tau + 4 * g4;
                const f32x4 sx = *reinterpret_cast<const f32x4*>(sSc + kScX * kC + r0);
                const f32x4 sb = *reinterpret_cast<const f32x4*>(sSc + kScBeta * kC + r0);
                const f32x4 vv = lds_tr4_f32(sV, SV, 16 * tau, wave * 16, g4, l16);
                Y[tau] = sb * (vv - sx * X[tau]);
            }
        }
        const bf16x8 yb0 = pack8(Y[0], Y[1]), yb1 = pack8(Y[2], Y[3]);
        // U = T Y   (T lower triangular: skip the all-zero upper k-step); T
        // is staged as row-operand fragments, one kilobyte each
        auto tfrag = [&](int tau, int ks) {
            if (!OUT) return ytf[ks == 0 ? tau : tau + 2];
            return *reinterpret_cast<const bf16x8*>(sT + 8 * ((tau * 2 + ks) * 64 + lane));
        };
        f32x4 U[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            U[tau] = mfma16(tfrag(tau, 0), yb0, f32x4{0.f, 0.f, 0.f, 0.f});
            if (tau >= 2) U[tau] = mfma16(tfrag(tau, 1), yb1, U[tau]);
        }
        if (OUT) {
            unsigned char* sU = lds + S::L_U + b * S::SZ_U;
            *reinterpret_cast<bf16x8*>(sU + cm_off<8>(16 * wave + l16, g4)) = pack8(U[0], U[1]);
            *reinterpret_cast<bf16x8*>(sU + cm_off<8>(16 * wave + l16, 4 + g4)) = pack8(U[2], U[3]);
        }
        // H' = exp(gamma_last) H + K^T diag(rk exp(gamma_last - gamma)) U
        f32x4 DU[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            const f32x4 sd = OUT ? *reinterpret_cast<const f32x4*>(sSc + kScD * kC + 16 * tau + 4 * g4) : ysd[tau];
            DU[tau] = sd * U[tau];
        }
        const bf16x8 db0 = pack8(DU[0], DU[1]), db1 = pack8(DU[2], DU[3]);
        const float e = sSc[kScE * kC];
#pragma unroll
        for (int mu = 0; mu < MT; ++mu) H[mu] *= e;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const bf16x8 db = kt ? db1 : db0;
#pragma unroll
            for (int m0 = 0; m0 < MT; m0 += 4) {
                bf16x8 at[4];
#pragma unroll
                for (int m = 0; m < 4 && m0 + m < MT; ++m) at[m] = kq_tr_pair<DK>(sK, 32 * kt, 16 * (m0 + m), g4, l16);
#pragma unroll
                for (int m = 0; m < 4 && m0 + m < MT; ++m) H[m0 + m] = mfma16(at[m], db, H[m0 + m]);
            }
        }
    };

    // ---------------- the pipeline ----------------
    // step s: compute waves run chunk s (buffer s & 1); helpers stage chunk
    // s + 1 into buffer (s + 1) & 1 and emit the outputs of chunk s - 1
    // (buffer (s - 1) & 1), whose q / P rows they loaded during step s - 1.
    // The two roles run separate loops with the same number of barriers.
    // An empty segment (a zero-length sequence) skips the pipeline entirely:
    // no wave meets a barrier and the state is only carried to the slot.
    const int steps = nch == 0 ? 0 : OUT ? nch + 1 : nch;
    if (helper) {
        if (steps == 0) return;
        HelperRows<KS> rows0, rows1 = {};   // rows1 feeds the first step's discarded outputs
        // In the state pass the helpers only stage, so their registers run a
        // step ahead of LDS: a step stages the chunk whose loads the previous
        // step issued, then issues the next chunk's loads, which then have a
        // whole step to arrive (the workspace rows often come from HBM). In
        // the output pass the emission between the loads and the staging
        // covers their latency.
        fetch(c0);
        if (OUT && sg.split) {
            // stage each transition the compute waves apply to reach this
            // segment's initial state (segments 2 and later), high and low
            // bf16 parts, swizzled like the k tiles, in LDS the pipeline has
            // not used yet
            constexpr int MP = 2 * DK * DK / 8 / S::NB;   // 16-byte pieces per helper thread
            for (int jh = 1; jh < sg.k; ++jh) {
                const uint16_t* mg = p.sm + (static_cast<size_t>(sg.g0 + jh) * p.hv + h) * (2 * DK * DK);
                u32x4 rm[MP];
#pragma unroll
                for (int m = 0; m < MP; ++m) rm[m] = *at_bytes<u32x4>(mg, 16u * (htid + S::NB * m));
                uint16_t* sM = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
                for (int m = 0; m < MP; ++m) {
                    const int e0 = 8 * (htid + S::NB * m);   // element of [2][DK][DK]
                    const int part = e0 / (DK * DK), rem = e0 - part * DK * DK;
                    const int r = rem / DK, cc = rem - r * DK;
                    *reinterpret_cast<u32x4*>(sM + part * DK * DK + kq_off<DK, false>(r, cc)) = rm[m];
                }
                lds_barrier();        // transition staged
                lds_barrier();        // compute waves done with it
            }
        }
        stage(0);
        if (!OUT) fetch(min(c0 + 1, c1 - 1));
        lds_barrier();
        u32x4 ov[OPL];
        auto hstep = [&](int s, int b, HelperRows<KS>& cur, HelperRows<KS>& nxt) {
            if (OUT) {
                fetch(min(c0 + s + 1, c1 - 1));
                fetch_rows(min(c0 + s, c1 - 1), nxt);
                emit_rows(b ^ 1, cur, ov);
                stage(b ^ 1);         // past the last chunk: a harmless copy into an unused buffer
                store_rows(c0 + max(s - 1, 0), s >= 1, ov);
            } else {
                stage(b ^ 1);
                fetch(min(c0 + s + 2, c1 - 1));
            }
            lds_barrier();
        };
        for (int s = 0; s < steps; s += 2) {
            hstep(s, 0, rows1, rows0);
            if (s + 1 < steps) hstep(s + 1, 1, rows0, rows1);
        }
        return;
    }
    // store this lane's state entries to a [DK][dv] fp32 tile through a
    // buffer resource: one lane offset and scalar row offsets (64-bit
    // per-element addresses would be hoisted out of the chunk loop and held in
    // registers for the whole pass)
    // (rows past `rows` fall outside the range and are dropped: pool tiles
    // have dkq rows, workspace tiles DK)
    auto store_tile = [&](float* tile, int rows) {
        const rsrc_t cr = make_rsrc(tile, 4u * rows * p.dv);
        const unsigned lo = 4u * (4 * g4 * p.dv + col);
#pragma unroll
        for (int mu = 0; mu < MT; ++mu)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(H[mu][i]), cr, lo,
                                                      4u * (16 * mu + i) * p.dv, 0);
    };
    // periodic checkpoint: the state after chunk c0 + s, when one is requested
    auto checkpoint = [&](int s) {
        if (!OUT || p.ckpt == nullptr) return;
        const int ck = p.ckpt[c0 + s];
        if (ck < 0) return;
        if (ck >= p.num_slots) {
            if (tid == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
            return;
        }
        store_tile(p.pool + (static_cast<size_t>(ck) * p.hv + h) * (static_cast<size_t>(p.dkq) * p.dv), p.dkq);
    };
    if (OUT && sg.split) {
        // segments 2 and later: H <- M_j H + E_j for the transitions of the
        // segments before this one (from the first segment's end state), as
        // bf16 MFMAs on high/low splits of both factors
        // (M_hi H_hi + M_hi H_lo + M_lo H_hi, about 16 significant bits)
        const uint16_t* sMh = reinterpret_cast<const uint16_t*>(lds);
        const uint16_t* sMl = sMh + DK * DK;
        for (int jh = 1; jh < sg.k; ++jh) {
            const float* se = p.se + (static_cast<size_t>(sg.g0 + jh) * p.hv + h) * (static_cast<size_t>(DK) * p.dv);
            f32x4 acc[MT];
#pragma unroll
            for (int mu = 0; mu < MT; ++mu)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mu][i] = se[(16 * mu + 4 * g4 + i) * p.dv + col];
            bf16x8 bh[KS], bl[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                f32x4 l0, l1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    l0[i] = H[2 * ks][i] - bf16_to_f32(f32_to_bf16(H[2 * ks][i]));
                    l1[i] = H[2 * ks + 1][i] - bf16_to_f32(f32_to_bf16(H[2 * ks + 1][i]));
                }
                bh[ks] = pack8(H[2 * ks], H[2 * ks + 1]);
                bl[ks] = pack8(l0, l1);
            }
            lds_barrier();            // transition staged
#pragma unroll
            for (int mu = 0; mu < MT; ++mu) {
                const int row = 16 * mu + l16;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 ah = kq_pair<DK, false>(sMh, row, 32 * ks, g4);
                    const bf16x8 al = kq_pair<DK, false>(sMl, row, 32 * ks, g4);
                    acc[mu] = mfma16(ah, bh[ks], acc[mu]);
                    acc[mu] = mfma16(ah, bl[ks], acc[mu]);
                    acc[mu] = mfma16(al, bh[ks], acc[mu]);
                }
            }
#pragma unroll
            for (int mu = 0; mu < MT; ++mu) H[mu] = acc[mu];
            lds_barrier();            // done with the transition
        }
    }
    // the state pass keeps a copy of a split sequence's initial state for the
    // output pass's first segment
    if (!OUT && sg.first) store_tile(p.sh + (static_cast<size_t>(blockIdx.y) * p.hv + h) * (static_cast<size_t>(DK) * p.dv), DK);
    if (steps > 0) lds_barrier();
    for (int s = 0; s < steps; s += 2) {
        if (s < nch) {
            chunk(0);
            checkpoint(s);
        }
        lds_barrier();
        if (s + 1 < steps) {
            if (s + 1 < nch) {
                chunk(1);
                checkpoint(s + 1);
            }
            lds_barrier();
        }
    }

    if (OUT) {
        if (!sg.last) return;               // a middle segment's end state is the next one's start (pass 2)
        store_tile(p.pool + (static_cast<size_t>(dsl) * p.hv + h) * (static_cast<size_t>(p.dkq) * p.dv), p.dkq);
    } else if (!m_cols) {
        store_tile(p.se + (static_cast<size_t>(blockIdx.y) * p.hv + h) * (static_cast<size_t>(DK) * p.dv), DK);
    } else {
        // transition M[d][m] (m = col), as bf16 high part and the bf16 rounding of the remainder
        uint16_t* out = p.sm + (static_cast<size_t>(blockIdx.y) * p.hv + h) * (2 * DK * DK);
#pragma unroll
        for (int mu = 0; mu < MT; ++mu)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = H[mu][i];
                const uint16_t hi = f32_to_bf16(x);
                const size_t e_off = static_cast<size_t>(16 * mu + 4 * g4 + i) * DK + col;
                out[e_off] = hi;
                out[DK * DK + e_off] = f32_to_bf16(x - bf16_to_f32(hi));
            }
    }
}

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked: ") + what + " launch failed: " + hipGetErrorString(e));
    return GDN_OK;
}

template <int DK, int MODE>
void launch_recurrence(const PrefillParams& p, int nw, int groups, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.hv * groups), static_cast<unsigned>(p.num_segs));
    switch (nw) {
        case 1: hipLaunchKernelGGL((prefill_recurrent_kernel<DK, 1, MODE>), grid, dim3(64 + 256), 0, s, p); break;
        case 2: hipLaunchKernelGGL((prefill_recurrent_kernel<DK, 2, MODE>), grid, dim3(128 + 256), 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_recurrent_kernel<DK, 4, MODE>), grid, dim3(256 + 256), 0, s, p); break;
    }
}

// float32 inputs: the intra-chunk kernel in its fp32 form, then the fp32
// recurrence (no sequence split)
template <int DK>
int launch_dk_f32(const PrefillParams& p, hipStream_t s) {
    if (p.num_chunks > 0) {
        hipLaunchKernelGGL((prefill_intra_kernel<DK, true>), dim3(p.num_chunks, p.hk), dim3(64), 0, s, p);
        const int st = check_launch("fp32 intra-chunk");
        if (st != GDN_OK) return st;
    }
    return launch_f32_recurrence(p, s);
}

template <int DK>
int launch_dk(const PrefillParams& p, int nw, hipStream_t s) {
    if (p.num_chunks > 0) {
        hipLaunchKernelGGL((prefill_intra_kernel<DK, false>), dim3(p.num_chunks, p.hk), dim3(64), 0, s, p);
        const int st = check_launch("intra-chunk");
        if (st != GDN_OK) return st;
    }
    const int groups = p.dv / (16 * nw);
    if (p.seg_len > 0) {
        // pass 1: every segment's local end state (value columns) and
        // transition (dk identity columns), all segments at once; its column
        // groups are at most dk wide so that the transition columns split
        // into whole groups
        const int nws = gdn::prefill_state_waves(DK, p.dv);
        launch_recurrence<DK, kModeState>(p, nws, p.dv / (16 * nws) + DK / (16 * nws), s);
        int st = check_launch("segment state pass");
        if (st != GDN_OK) return st;
    }
    launch_recurrence<DK, kModeOutput>(p, nw, groups, s);
    return check_launch("recurrence");
}

}  // namespace

namespace gdn {

int launch_prefill(const gdn_pool* pool, const gdn_prefill_args* a, const PrefillPlan& plan, void* workspace,
                   void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    PrefillParams p;
    p.cu = a->cu_seqlens;
    p.chunk_off = reinterpret_cast<const int32_t*>(ws + plan.off_chunk_offsets);
    p.chunk_off_w = reinterpret_cast<int32_t*>(ws + plan.off_chunk_offsets);
    p.q = static_cast<const uint16_t*>(a->q);
    p.k = static_cast<const uint16_t*>(a->k);
    p.v = static_cast<const uint16_t*>(a->v);
    p.g = a->g;
    p.beta = a->beta;
    p.o = static_cast<uint16_t*>(a->o);
    p.qf = static_cast<const float*>(a->q);
    p.kf = static_cast<const float*>(a->k);
    p.vf = static_cast<const float*>(a->v);
    p.of = static_cast<float*>(a->o);
    p.tpf = reinterpret_cast<float*>(ws + plan.off_tp);
    p.pool = pool->storage;
    p.src = a->src_slots;
    p.dst = a->dst_slots;
    p.err = a->err_flag;
    p.ckpt = a->ckpt_slots;
    p.tp = reinterpret_cast<uint16_t*>(ws + plan.off_tp);
    p.sc = reinterpret_cast<float*>(ws + plan.off_sc);
    p.seg_off = reinterpret_cast<const int32_t*>(ws + plan.off_seg_offsets);
    p.seg_off_w = reinterpret_cast<int32_t*>(ws + plan.off_seg_offsets);
    p.se = reinterpret_cast<float*>(ws + plan.off_se);
    p.sm = reinterpret_cast<uint16_t*>(ws + plan.off_sm);
    p.sh = reinterpret_cast<float*>(ws + plan.off_sh);
    p.seg_len = plan.seg_len;
    p.num_segs = plan.num_segs;
    p.n_seqs = a->num_seqs;
    p.num_chunks = plan.num_chunks;
    p.total_tokens = a->total_tokens;
    p.hk = a->num_k_heads;
    p.hv = a->num_v_heads;
    p.group = a->num_v_heads / a->num_k_heads;
    p.dkq = a->dk;
    p.dv = a->dv;
    p.num_slots = pool->num_slots;
    p.scale = a->scale;
    p.eps = a->l2_eps;

    p.inl_n = 0;
    if (a->num_seqs <= kInlineSeqs) {
        // first chunk and first segment of every sequence from the host
        // mirror of cu_seqlens, as the planner counted them
        int32_t cc = 0, ss = 0;
        for (int32_t i = 0; i < a->num_seqs; ++i) {
            p.inl_chunk[i] = cc;
            p.inl_seg[i] = ss;
            const int32_t len = a->cu_seqlens_host[i + 1] - a->cu_seqlens_host[i];
            const int32_t nc = len > 0 ? (len + kC - 1) / kC : 0;
            cc += nc;
            ss += (plan.seg_len == 0 || nc <= plan.seg_len) ? 1 : (nc + plan.seg_len - 1) / plan.seg_len;
        }
        p.inl_chunk[a->num_seqs] = cc;
        p.inl_seg[a->num_seqs] = ss;
        p.inl_n = a->num_seqs;
    } else {
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(kOffThreads), 0, s, p);
        const int st = check_launch("chunk-offset");
        if (st != GDN_OK) return st;
    }
    if (a->dtype == GDN_DTYPE_F32) {
        switch (a->dk) {
            case 16: return launch_dk_f32<16>(p, s);
            case 32: return launch_dk_f32<32>(p, s);
            case 64: return launch_dk_f32<64>(p, s);
            case 128: return launch_dk_f32<128>(p, s);
            default: return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: unsupported dk");
        }
    }
    const int nw = prefill_output_waves(a->dv);
    switch (prefill_kernel_dk(a->dk)) {
        case 32: return launch_dk<32>(p, nw, s);
        case 64: return launch_dk<64>(p, nw, s);
        case 128: return launch_dk<128>(p, nw, s);
        default: return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: unsupported dk");
    }
}

}  // namespace gdn
