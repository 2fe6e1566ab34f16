// HIP kernels of the chunked gated delta rule forward pass, written for
// gfx950 (CDNA4: wave64, bf16 MFMA 16x16x32 / 16x16x16, 160 KiB LDS per CU).
//
// The op is `chunk_gated_delta_rule` with chunk size 64 and a varlen
// cu_seqlens API ("FlashQLA GDN backend produces different tokens from FLA
// Triton", Setup).  Per sequence and v-head the state H = S^T (dk x dv) obeys
// the gated delta rule S_t = exp(g_t) S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = scale S_t q_t.  Within a 64-token chunk with incoming state H0 and
// chunk-local gate prefix sums G (all exponents below are <= 0):
//
//   A_ij  = b_i exp(G_i - G_j) (k_i . k_j)    for j < i
//   [W|U] = (I + A)^-1 [diag(b e^G) K | diag(b) V]        (the WY form)
//   Vnew  = U - W H0
//   O     = scale (diag(e^G) Q H0 + P Vnew),  P_ij = exp(G_i - G_j) (q_i . k_j), j <= i
//   H     = e^{G_L} H0 + K^T diag(e^{G_L - G}) Vnew
//
// Kernels:
//   gdr_prepare_kernel  chunk offsets / chunk map / longest-first sequence
//                       order, derived from the cu_seqlens content on the
//                       device on every call ("Findings from integrating
//                       FlashQLA's Blackwell GDN kernels into a JAX trainer",
//                       item 1: no identity-keyed cache).
//   gdr_cumsum_kernel   chunk-local inclusive prefix sum of the log-gate.
//   gdr_fwd_kernel      the whole chunk pipeline fused: one work-group walks
//                       one (sequence, v-head) through its chunks in order with
//                       the fp32 state in MFMA accumulator registers.
//
// MFMA operand layout used throughout (16x16 tiles, lane l, l16 = l % 16,
// lq = l / 16, r = 0..3):
//   A fragment (rows x k):  row l16, k = 4*lq + r
//   B fragment (k x cols):  col l16, k = 4*lq + r
//   C/D tile:               col l16, row = 4*lq + r
// so an MFMA result tile is directly the B fragment of the next product over
// its rows.  Every product runs on the 16x16x32 instruction used as two
// 16x16x16 products fused: lane slots 0-3 carry one K16 block and slots 4-7
// the next one, the same pairing on both operands (the instruction's own k
// numbering of the slots does not matter because it is shared by A and B).
// A lone K16 block is zero-padded rather than issued as a 16x16x16
// instruction: chaining a 16x16x16 accumulation on the result of a 16x16x32
// one was observed to read a partly written accumulator on gfx950.
#include "gdr_internal.h"

#include <stdint.h>

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// one K16 block on the 16x16x32 instruction, upper slots zero
__device__ __forceinline__ f32x4 mfma16z(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16x4 z = {};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   c, 0, 0, 0);
}
// the 16x16x16 instruction, for the lane-layout self test only
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 ld4(const uint16_t *p) {   // 8-byte LDS read
    return *reinterpret_cast<const bf16x4 *>(p);
}
__device__ __forceinline__ bf16x4 cvt4(f32x4 x) {           // round to nearest even
    bf16x4 r;
    r[0] = (__bf16)x[0];
    r[1] = (__bf16)x[1];
    r[2] = (__bf16)x[2];
    r[3] = (__bf16)x[3];
    return r;
}
__device__ __forceinline__ f32x4 up4(bf16x4 x) {
    f32x4 r;
    r[0] = (float)x[0];
    r[1] = (float)x[1];
    r[2] = (float)x[2];
    r[3] = (float)x[3];
    return r;
}
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <bool BF16>
__device__ __forceinline__ float load_scalar(const void *p, int64_t i) {
    if constexpr (BF16) {
        const uint16_t u = reinterpret_cast<const uint16_t *>(p)[i];
        return __uint_as_float(static_cast<uint32_t>(u) << 16);
    } else {
        return reinterpret_cast<const float *>(p)[i];
    }
}

// 8 consecutive elements of a row as 8 bf16 (16 bytes); f32 inputs are rounded.
template <bool BF16>
__device__ __forceinline__ uint4 load8(const void *p, int64_t i) {
    if constexpr (BF16) {
        return *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p) + i);
    } else {
        const float4 x = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
        const float4 y = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i + 4);
        uint4 r;
        r.x = bf16_bits(x.x) | (static_cast<uint32_t>(bf16_bits(x.y)) << 16);
        r.y = bf16_bits(x.z) | (static_cast<uint32_t>(bf16_bits(x.w)) << 16);
        r.z = bf16_bits(y.x) | (static_cast<uint32_t>(bf16_bits(y.y)) << 16);
        r.w = bf16_bits(y.z) | (static_cast<uint32_t>(bf16_bits(y.w)) << 16);
        return r;
    }
}

__device__ __forceinline__ uint16_t elem8(const uint4 &v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// --------------------------------------------------------------------------
// Fused forward: LDS layout of one work-group (bf16 buffers hold raw bits).
// --------------------------------------------------------------------------
template <int D>
struct FwdLds {
    static constexpr int PK = D + 8;   // pitch of [64][D] row-major buffers (q, k, -W)
    static constexpr int PT = C + 8;   // pitch of [D][64] transposed buffers (k^T, v^T)
    static constexpr int PP = C + 8;   // pitch of P [64][64]
    static constexpr int PA = C + 4;   // pitch of A [64][64] (f32)
    static constexpr int PD = 20;      // pitch of the four 16x16 diagonal inverses (f32)
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + C * PK * 2;
    static constexpr int oW = oK + C * PK * 2;
    static constexpr int oKT = oW + C * PK * 2;
    static constexpr int oVT = oKT + D * PT * 2;
    static constexpr int oP = oVT + D * PT * 2;
    static constexpr int oA = oP + C * PP * 2;
    static constexpr int oDi = oA + C * PA * 4;
    static constexpr int oS = oDi + 4 * 16 * PD * 4;   // six [64] f32 vectors
    static constexpr int bytes = oS + 6 * C * 4;
};

// Lower-triangular 16x16 tile pairs (ib >= jb) of a 64x64 chunk matrix.
__constant__ int8_t kTileI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <int D, bool IN_BF16, bool GATE_BF16>
__global__ void __launch_bounds__(kFwdThreads, 1) gdr_fwd_kernel(FwdArgs a) {
    using Ly = FwdLds<D>;
    constexpr int PK = Ly::PK, PT = Ly::PT, PP = Ly::PP, PA = Ly::PA, PD = Ly::PD;
    constexpr int DW = D / 4;      // dv columns owned by each of the 4 waves
    constexpr int NTW = DW / 16;   // 16-wide column tiles per wave
    constexpr int KB = D / 16;     // K16 blocks over the head dim
    static_assert(KB % 2 == 0, "head dim must be a multiple of 32");

    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(smem + Ly::oQ);
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem + Ly::oK);
    uint16_t *sW = reinterpret_cast<uint16_t *>(smem + Ly::oW);
    uint16_t *sKT = reinterpret_cast<uint16_t *>(smem + Ly::oKT);
    uint16_t *sVT = reinterpret_cast<uint16_t *>(smem + Ly::oVT);
    uint16_t *sP = reinterpret_cast<uint16_t *>(smem + Ly::oP);
    float *sA = reinterpret_cast<float *>(smem + Ly::oA);
    float *sDi = reinterpret_cast<float *>(smem + Ly::oDi);
    float *sG2 = reinterpret_cast<float *>(smem + Ly::oS);   // G * log2(e)
    float *sB = sG2 + C;                                     // beta
    float *sBG = sB + C;                                     // beta * e^G
    float *sGam = sBG + C;                                   // e^G
    float *sDec = sGam + C;                                  // e^{G_last - G}
    float *sMisc = sDec + C;                                 // [0] = e^{G_last}

    // ---- work item: (sequence n, v-head h), longest sequences first
    const int64_t item = blockIdx.x;
    const int64_t rank = item / a.hv;
    const int h = static_cast<int>(item % a.hv);
    const int64_t n = a.order ? static_cast<int64_t>(a.order[rank]) : rank;
    if (n < 0 || n >= a.n_seq) return;
    int64_t bos, eos;
    if (a.cu) {
        bos = a.cu[n];
        eos = a.cu[n + 1];
    } else {
        bos = n * a.seq_len;
        eos = bos + a.seq_len;
    }
    bos = bos < 0 ? 0 : bos;
    eos = eos > a.total_tokens ? a.total_tokens : eos;
    if (eos <= bos) return;   // length-0 segment: reads nothing, writes nothing
    const int hk = h / (a.hv / a.hk);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lq = lane >> 4;
    const int colw = wave * DW;   // first dv column of this wave

    // ---- fp32 state in C layout: tile (kb, nt) holds rows dk 16kb+4lq+r, column dv colw+16nt+l16
    f32x4 hs[KB][NTW];
    const int64_t sbase = (n * a.hv + h) * static_cast<int64_t>(D) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                hs[kb][nt][r] = a.h0 ? a.h0[sbase + (16 * kb + 4 * lq + r) * D + colw + 16 * nt + l16] : 0.f;

    const int64_t nchunks = (eos - bos + C - 1) / C;
    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t t0 = bos + ci * C;
        const int L = static_cast<int>((eos - t0) < C ? (eos - t0) : C);

        // ---- stage q, k (row-major) and k, v (transposed) of this chunk in LDS
        {
            constexpr int FG = D / 8;        // 8-element feature groups per row
            constexpr int TG = 256 / FG;     // token groups
            constexpr int TPT = C / TG;      // tokens per thread (4 at D=128, 2 at D=64)
            const int fg = tid % FG, tg = tid / FG;
            const int f0 = fg * 8;
            uint4 qv[TPT], kv[TPT], vv[TPT];
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const int t = tg * TPT + j;
                if (t < L) {
                    const int64_t tok = t0 + t;
                    qv[j] = load8<IN_BF16>(a.q, (tok * a.hk + hk) * D + f0);
                    kv[j] = load8<IN_BF16>(a.k, (tok * a.hk + hk) * D + f0);
                    vv[j] = load8<IN_BF16>(a.v, (tok * a.hv + h) * D + f0);
                } else {
                    qv[j] = kv[j] = vv[j] = make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const int t = tg * TPT + j;
                *reinterpret_cast<uint4 *>(sQ + t * PK + f0) = qv[j];
                *reinterpret_cast<uint4 *>(sK + t * PK + f0) = kv[j];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (TPT == 4) {
                    uint2 kt, vt;
                    kt.x = elem8(kv[0], e) | (static_cast<uint32_t>(elem8(kv[1], e)) << 16);
                    kt.y = elem8(kv[2], e) | (static_cast<uint32_t>(elem8(kv[3], e)) << 16);
                    vt.x = elem8(vv[0], e) | (static_cast<uint32_t>(elem8(vv[1], e)) << 16);
                    vt.y = elem8(vv[2], e) | (static_cast<uint32_t>(elem8(vv[3], e)) << 16);
                    *reinterpret_cast<uint2 *>(sKT + (f0 + e) * PT + tg * TPT) = kt;
                    *reinterpret_cast<uint2 *>(sVT + (f0 + e) * PT + tg * TPT) = vt;
                } else {
                    static_assert(TPT == 2, "unsupported head dim");
                    *reinterpret_cast<uint32_t *>(sKT + (f0 + e) * PT + tg * TPT) =
                        elem8(kv[0], e) | (static_cast<uint32_t>(elem8(kv[1], e)) << 16);
                    *reinterpret_cast<uint32_t *>(sVT + (f0 + e) * PT + tg * TPT) =
                        elem8(vv[0], e) | (static_cast<uint32_t>(elem8(vv[1], e)) << 16);
                }
            }
        }
        // ---- gates: chunk-local prefix sum of g, one token per lane of wave 0
        if (wave == 0) {
            float gv = 0.f, bv = 0.f;
            if (lane < L) {
                const int64_t gi = (t0 + lane) * a.hv + h;
                gv = load_scalar<GATE_BF16>(a.g, gi);
                bv = load_scalar<GATE_BF16>(a.beta, gi);
            }
            const float G2 = wave_inclusive_scan(gv, lane) * kLog2e;
            const float Glast2 = __shfl(G2, 63, 64);   // padding has g = 0: equals G at L-1
            const float gam = exp2f(G2);
            sG2[lane] = G2;
            sB[lane] = bv;
            sBG[lane] = bv * gam;
            sGam[lane] = gam;
            sDec[lane] = exp2f(Glast2 - G2);
            if (lane == 0) sMisc[0] = exp2f(Glast2);
        }
        __syncthreads();

        // ---- A = strictly lower part of diag(b) (e^{G_i - G_j}) o K K^T   (f32, LDS)
        for (int ti = wave; ti < 10; ti += 4) {
            const int ib = kTileI[ti], jb = kTileJ[ti];
            f32x4 acc = zero4();
            const uint16_t *pa = sK + (16 * jb + l16) * PK + 4 * lq;
            const uint16_t *pb = sK + (16 * ib + l16) * PK + 4 * lq;
#pragma unroll
            for (int p = 0; p < KB / 2; ++p)
                acc = mfma32(cat(ld4(pa + 32 * p), ld4(pa + 32 * p + 16)),
                             cat(ld4(pb + 32 * p), ld4(pb + 32 * p + 16)), acc);
            // tile element (row j, col i) = k_j . k_i
            const int i = 16 * ib + l16;
            const float gi = sG2[i], bi = sB[i];
            f32x4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jb + 4 * lq + r;
                out[r] = (i > j) ? bi * exp2f(gi - sG2[j]) * acc[r] : 0.f;
            }
            *reinterpret_cast<f32x4 *>(sA + i * PA + 16 * jb + 4 * lq) = out;
        }
        __syncthreads();

        if (wave == 0) {
            // ---- inverses of the four 16x16 unit lower diagonal blocks of I + A
            // lane = (block, column): forward substitution down the column
            const int blk = lane >> 4, c = l16;
            const float *Ab = sA + (16 * blk) * PA + 16 * blk;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s -= Ab[i * PA + j] * x[j];
                x[i] = s;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sDi[(16 * blk + i) * PD + c] = x[i];
        } else {
            // ---- P = lower part of (e^{G_i - G_j}) o Q K^T   (bf16, LDS)
            for (int ti = wave - 1; ti < 10; ti += 3) {
                const int ib = kTileI[ti], jb = kTileJ[ti];
                f32x4 acc = zero4();
                const uint16_t *pa = sK + (16 * jb + l16) * PK + 4 * lq;   // keys
                const uint16_t *pb = sQ + (16 * ib + l16) * PK + 4 * lq;   // queries
#pragma unroll
                for (int p = 0; p < KB / 2; ++p)
                    acc = mfma32(cat(ld4(pa + 32 * p), ld4(pa + 32 * p + 16)),
                                 cat(ld4(pb + 32 * p), ld4(pb + 32 * p + 16)), acc);
                // tile element (row j = key, col i = query) = k_j . q_i
                const int i = 16 * ib + l16;
                const float gi = sG2[i];
                f32x4 out;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jb + 4 * lq + r;
                    out[r] = (i >= j) ? exp2f(gi - sG2[j]) * acc[r] : 0.f;
                }
                *reinterpret_cast<bf16x4 *>(sP + i * PP + 16 * jb + 4 * lq) = cvt4(out);
            }
        }
        __syncthreads();

        // ---- WY solve by 16-row blocks: X_a = D_a (B_a - sum_{c<a} A_ac X_c)
        // tiles tt < NTW: W columns (dk) colw+16tt..; tt >= NTW: U columns (dv)
        bf16x4 Xb[4][2 * NTW];
        f32x4 U[4][NTW];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int trow = 16 * blk + 4 * lq;
            const f32x4 bg = *reinterpret_cast<const f32x4 *>(sBG + trow);
            const f32x4 bb = *reinterpret_cast<const f32x4 *>(sB + trow);
            f32x4 R[2 * NTW];
#pragma unroll
            for (int tt = 0; tt < 2 * NTW; ++tt) {
                const bool isW = tt < NTW;
                const int col = colw + 16 * (isW ? tt : tt - NTW) + l16;
                const f32x4 raw = up4(ld4((isW ? sKT : sVT) + col * PT + trow));
                R[tt] = raw * (isW ? bg : bb);
            }
            const float *arow = sA + (16 * blk + l16) * PA + 4 * lq;
#pragma unroll
            for (int c = 0; c + 1 < blk; c += 2) {
                const bf16x8 af = cat(cvt4(-*reinterpret_cast<const f32x4 *>(arow + 16 * c)),
                                      cvt4(-*reinterpret_cast<const f32x4 *>(arow + 16 * c + 16)));
#pragma unroll
                for (int tt = 0; tt < 2 * NTW; ++tt)
                    R[tt] = mfma32(af, cat(Xb[c][tt], Xb[c + 1][tt]), R[tt]);
            }
            if (blk & 1) {
                const int c = blk - 1;
                const bf16x4 af = cvt4(-*reinterpret_cast<const f32x4 *>(arow + 16 * c));
#pragma unroll
                for (int tt = 0; tt < 2 * NTW; ++tt) R[tt] = mfma16z(af, Xb[c][tt], R[tt]);
            }
            const bf16x4 df = cvt4(*reinterpret_cast<const f32x4 *>(sDi + (16 * blk + l16) * PD + 4 * lq));
#pragma unroll
            for (int tt = 0; tt < 2 * NTW; ++tt) {
                const f32x4 X = mfma16z(df, cvt4(R[tt]), zero4());
                Xb[blk][tt] = cvt4(X);
                if (tt < NTW) {
                    const int col = colw + 16 * tt + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sW[(trow + r) * PK + col] = bf16_bits(-X[r]);
                } else {
                    U[blk][tt - NTW] = X;
                }
            }
        }
        __syncthreads();

        // ---- Vnew = U - W H0   (sW holds -W)
        bf16x4 hb[KB][NTW];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) hb[kb][nt] = cvt4(hs[kb][nt]);
        f32x4 Vn[4][NTW];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) Vn[blk][nt] = U[blk][nt];
            const uint16_t *pw = sW + (16 * blk + l16) * PK + 4 * lq;
#pragma unroll
            for (int p = 0; p < KB / 2; ++p) {
                const bf16x8 af = cat(ld4(pw + 32 * p), ld4(pw + 32 * p + 16));
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    Vn[blk][nt] = mfma32(af, cat(hb[2 * p][nt], hb[2 * p + 1][nt]), Vn[blk][nt]);
            }
        }

        // ---- O = scale (diag(e^G) Q H0 + P Vnew)
        bf16x4 Vb[4][NTW];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) Vb[blk][nt] = cvt4(Vn[blk][nt]);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4 oacc[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) oacc[nt] = zero4();
            const uint16_t *pq = sQ + (16 * blk + l16) * PK + 4 * lq;
#pragma unroll
            for (int p = 0; p < KB / 2; ++p) {
                const bf16x8 af = cat(ld4(pq + 32 * p), ld4(pq + 32 * p + 16));
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    oacc[nt] = mfma32(af, cat(hb[2 * p][nt], hb[2 * p + 1][nt]), oacc[nt]);
            }
            const int trow = 16 * blk + 4 * lq;
            const f32x4 gam = *reinterpret_cast<const f32x4 *>(sGam + trow);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) oacc[nt] = oacc[nt] * gam;
            const uint16_t *pp = sP + (16 * blk + l16) * PP + 4 * lq;
#pragma unroll
            for (int c = 0; c + 1 <= blk; c += 2) {
                const bf16x8 pf = cat(ld4(pp + 16 * c), ld4(pp + 16 * c + 16));
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    oacc[nt] = mfma32(pf, cat(Vb[c][nt], Vb[c + 1][nt]), oacc[nt]);
            }
            if ((blk & 1) == 0) {
                const bf16x4 pf = ld4(pp + 16 * blk);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) oacc[nt] = mfma16z(pf, Vb[blk][nt], oacc[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int col = colw + 16 * nt + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = trow + r;
                    if (t < L) {
                        const int64_t oi = ((t0 + t) * a.hv + h) * D + col;
                        const float val = a.scale * oacc[nt][r];
                        if constexpr (IN_BF16)
                            reinterpret_cast<uint16_t *>(a.o)[oi] = bf16_bits(val);
                        else
                            reinterpret_cast<float *>(a.o)[oi] = val;
                    }
                }
            }
        }

        // ---- H = e^{G_L} H0 + K^T diag(e^{G_L - G}) Vnew
        {
            const float gl = sMisc[0];
            bf16x4 Vt[4][NTW];
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const f32x4 dec = *reinterpret_cast<const f32x4 *>(sDec + 16 * blk + 4 * lq);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) Vt[blk][nt] = cvt4(Vn[blk][nt] * dec);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const uint16_t *pk = sKT + (16 * kb + l16) * PT + 4 * lq;
                const bf16x8 a01 = cat(ld4(pk), ld4(pk + 16));
                const bf16x8 a23 = cat(ld4(pk + 32), ld4(pk + 48));
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    f32x4 s = hs[kb][nt] * gl;
                    s = mfma32(a01, cat(Vt[0][nt], Vt[1][nt]), s);
                    s = mfma32(a23, cat(Vt[2][nt], Vt[3][nt]), s);
                    hs[kb][nt] = s;
                }
            }
        }
        __syncthreads();   // LDS is restaged by the next chunk
    }

    if (a.ht) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.ht[sbase + (16 * kb + 4 * lq + r) * D + colw + 16 * nt + l16] = hs[kb][nt][r];
    }
}

// --------------------------------------------------------------------------
// Chunk indices from cu_seqlens (one work-group of 1024 threads)
// --------------------------------------------------------------------------
constexpr int kPrepThreads = 1024;
constexpr int kSortMax = 8192;

__global__ void __launch_bounds__(kPrepThreads) gdr_prepare_kernel(
    const int32_t *cu, int64_t n_seq, int32_t *offs, int32_t *map, int64_t nt_max, int32_t *order) {
    __shared__ int32_t s_scan[kPrepThreads];
    __shared__ int32_t s_len[kSortMax];
    const int tid = threadIdx.x;
    int64_t carry = 0;
    for (int64_t base = 0; base < n_seq; base += kPrepThreads) {
        const int64_t n = base + tid;
        int32_t len = 0;
        if (n < n_seq) {
            len = cu[n + 1] - cu[n];
            len = len < 0 ? 0 : len;
        }
        const int32_t nc = (len + C - 1) / C;
        s_scan[tid] = nc;
        __syncthreads();
        for (int off = 1; off < kPrepThreads; off <<= 1) {
            const int32_t y = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += y;
            __syncthreads();
        }
        const int64_t excl = carry + s_scan[tid] - nc;
        if (n < n_seq) {
            if (offs) offs[n] = static_cast<int32_t>(excl);
            if (map)
                for (int32_t c = 0; c < nc; ++c) {
                    const int64_t i = excl + c;
                    if (i < nt_max) {
                        map[2 * i] = static_cast<int32_t>(n);
                        map[2 * i + 1] = c;
                    }
                }
            if (n < kSortMax) s_len[n] = len;
        }
        carry += s_scan[kPrepThreads - 1];
        __syncthreads();
    }
    if (tid == 0 && offs) offs[n_seq] = static_cast<int32_t>(carry);
    if (map)
        for (int64_t i = carry + tid; i < nt_max; i += kPrepThreads) {
            map[2 * i] = -1;
            map[2 * i + 1] = -1;
        }
    if (order) {
        if (n_seq <= kSortMax) {
            for (int64_t n = tid; n < n_seq; n += kPrepThreads) {
                const int32_t ln = s_len[n];
                int64_t rank = 0;
                for (int64_t m = 0; m < n_seq; ++m) {
                    const int32_t lm = s_len[m];
                    rank += (lm > ln) || (lm == ln && m < n);
                }
                order[rank] = static_cast<int32_t>(n);
            }
        } else {
            for (int64_t n = tid; n < n_seq; n += kPrepThreads) order[n] = static_cast<int32_t>(n);
        }
    }
}

// --------------------------------------------------------------------------
// Chunk-local prefix sum of the log-gate, one work-group (4 waves) per chunk
// --------------------------------------------------------------------------
template <bool GATE_BF16>
__global__ void __launch_bounds__(256) gdr_cumsum_kernel(const void *g, const int32_t *cu,
                                                          const int32_t *map, int64_t n_rows,
                                                          int64_t seq_len, int64_t total_tokens,
                                                          int32_t heads, float *G) {
    int64_t bos, len, c;
    if (map) {
        const int32_t n = map[2 * blockIdx.x];
        if (n < 0) return;
        c = map[2 * blockIdx.x + 1];
        bos = cu[n];
        len = static_cast<int64_t>(cu[n + 1]) - bos;
    } else {
        const int64_t per = (seq_len + C - 1) / C;
        const int64_t row = blockIdx.x / per;
        if (row >= n_rows) return;
        c = blockIdx.x % per;
        bos = row * seq_len;
        len = seq_len;
    }
    const int64_t t0 = bos + C * c;
    int64_t L = len - C * c;
    L = L > C ? C : L;
    if (t0 < 0 || L <= 0) return;
    if (t0 + L > total_tokens) L = total_tokens - t0;
    if (L <= 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int hh = wave; hh < heads; hh += 4) {
        const float x = lane < L ? load_scalar<GATE_BF16>(g, (t0 + lane) * heads + hh) : 0.f;
        const float s = wave_inclusive_scan(x, lane);
        if (lane < L) G[(t0 + lane) * heads + hh] = s;
    }
}

// --------------------------------------------------------------------------
// MFMA lane-layout self test: one wave, both bf16 shapes the kernels use
// --------------------------------------------------------------------------
__global__ void __launch_bounds__(64) gdr_selftest_kernel(const uint16_t *a, const uint16_t *b, float *c) {
    const int l = threadIdx.x;
    bf16x8 av, bv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        av[i] = __builtin_bit_cast(__bf16, a[8 * l + i]);
        bv[i] = __builtin_bit_cast(__bf16, b[8 * l + i]);
    }
    const f32x4 c0 = mfma32(av, bv, zero4());
    const f32x4 c1 = mfma16(__builtin_shufflevector(av, av, 0, 1, 2, 3),
                            __builtin_shufflevector(bv, bv, 0, 1, 2, 3), zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        c[4 * l + r] = c0[r];
        c[256 + 4 * l + r] = c1[r];
    }
}

template <int D, bool IN_BF16, bool GATE_BF16>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t stream) {
    auto kern = gdr_fwd_kernel<D, IN_BF16, GATE_BF16>;
    const int lds = FwdLds<D>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.n_seq * a.hv)), dim3(kFwdThreads), lds,
                       stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs &a, hipStream_t s) {
    if (a.in_bf16) return a.gate_bf16 ? launch_fwd_t<D, true, true>(a, s) : launch_fwd_t<D, true, false>(a, s);
    return a.gate_bf16 ? launch_fwd_t<D, false, true>(a, s) : launch_fwd_t<D, false, false>(a, s);
}

}  // namespace

int fwd_lds_bytes(int d) { return d == 64 ? FwdLds<64>::bytes : FwdLds<128>::bytes; }

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
    if (a.n_seq == 0 || a.hv == 0) return hipSuccess;
    return a.d == 64 ? launch_fwd_d<64>(a, stream) : launch_fwd_d<128>(a, stream);
}

hipError_t launch_prepare(const int32_t *cu, int64_t n_seq, int32_t *chunk_offsets, int32_t *chunk_map,
                          int64_t nt_max, int32_t *order, hipStream_t stream) {
    hipLaunchKernelGGL(gdr_prepare_kernel, dim3(1), dim3(kPrepThreads), 0, stream, cu, n_seq,
                       chunk_offsets, chunk_map, nt_max, order);
    return hipGetLastError();
}

hipError_t launch_cumsum(const void *g, int gate_bf16, const int32_t *cu, const int32_t *chunk_map,
                         int64_t nt_max, int64_t n_rows, int64_t seq_len, int64_t total, int32_t heads,
                         float *G, hipStream_t stream) {
    const int64_t grid = chunk_map ? nt_max : n_rows * ((seq_len + C - 1) / C);
    if (grid == 0 || heads == 0) return hipSuccess;
    if (gate_bf16)
        hipLaunchKernelGGL(gdr_cumsum_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                           g, cu, chunk_map, n_rows, seq_len, total, heads, G);
    else
        hipLaunchKernelGGL(gdr_cumsum_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                           g, cu, chunk_map, n_rows, seq_len, total, heads, G);
    return hipGetLastError();
}

hipError_t launch_selftest_mfma(const uint16_t *a, const uint16_t *b, float *c, hipStream_t stream) {
    hipLaunchKernelGGL(gdr_selftest_kernel, dim3(1), dim3(64), 0, stream, a, b, c);
    return hipGetLastError();
}

}  // namespace gdr
