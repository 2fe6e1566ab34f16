// HIP kernels of the backward pass of the chunked gated delta rule, for
// gfx950 (CDNA4).  The pages treat the backward as the other half of the
// FlashQLA kernel family ("Findings from integrating FlashQLA's Blackwell GDN
// kernels into a JAX trainer": opening summary, items 3-4); they give no
// formula, so the gradients here are the reverse-mode derivative of the
// forward recurrence written in chunk form.
//
// One chunk of 64 tokens (rows past the sequence end are zero with g = b = 0),
// state S (= H, dk x dv) at its start, G the chunk-local prefix sum of g,
// gamma = e^G, lambda = e^{G_L - G}, A~_ij = e^{G_i - G_j} k_i.k_j (j < i),
// T = (I + diag(b) A~)^-1, M_ij = e^{G_i - G_j} (j <= i).  Forward:
//
//   X = K S,  R~ = V - diag(gamma) X,  U = T diag(b) R~
//   O = scale (diag(gamma) Q S + (M o Q K^T) U)
//   S' = e^{G_L} S + K^T diag(lambda) U
//
// Given dO and dS' (the gradient of the state at the chunk end):
//
//   dU  = scale (M o Q K^T)^T dO + diag(lambda) K dS'      (local part dU0 + chain part)
//   dW  = T^T dU,   dV = diag(b) dW
//   dS  = e^{G_L} dS' + scale Q^T diag(gamma) dO - w^T dU,  w = T diag(b gamma) K
//   Zs  = scale M o (dO U^T),   dBn = -(strictly lower M) o (dW U^T),   dB = diag(b) dBn
//   dQ  = scale diag(gamma) dO S^T + Zs K
//   dK  = [-diag(b gamma) dW S^T + diag(b) dBn K]              (row uses of k)
//       + [diag(lambda) U dS'^T + Zs^T Q + dB^T K]              (column uses of k)
//   db  = rowsum(dW o R~) + rowsum(K o (dBn K))
//   dG  = rowsum(Q o dQ) + rowsum(K o row part) - rowsum(K o column part),
//         plus, in the last row, e^{G_L} <dS', S> + sum_j lambda_j k_j . (U dS'^T)_j
//   dg  = reverse prefix sum of dG within the chunk
//
// The gate enters every term as e^{G_i} on a row and e^{-G_j} on a column, so
// its gradient is q.dq + k.(row part) - k.(column part) (plus the G_L terms).
// q and k gradients of the v-heads that share a q/k head add up.
//
// Kernels (after the forward kernel has written the state after every chunk):
//   gdr_bwd_prep_kernel   per (chunk, v-head pair of one q/k head, or one
//                         v-head), in parallel: T by block substitution.
//   gdr_bwd_chain_kernel  per (sequence, v-head), chunks in reverse order:
//                         dS' kept in fp32 registers, dU = dU0 + its chain
//                         part (dU0 and w formed in the chain from q, k, dO
//                         and T),
//                         dS' of every chunk stored for the next kernel.
//   gdr_bwd_grads_kernel  per (chunk, q/k head), in parallel, looping over the
//                         v-heads of the group: dq, dk, dv, dg, dbeta.
#include "gdr_internal.h"
#include "gdr_device.h"

#include <stdint.h>

namespace gdr {
namespace {

constexpr int kBwdThreads = 512;     // prep and gradient kernels: 8 waves
constexpr int kChainThreads = 256;   // reverse chain: 4 waves

// A fragment from [m][k] storage (or a B fragment from [n][k] storage): rows
// row0 + l16, k = k0 + 16 h + 4 lq + r for the two K16 halves h.
__device__ __forceinline__ bf16x8 frag_rows(const uint16_t *M, int pitch, int row0, int k0, int l16, int lq) {
    const uint16_t *p = M + (row0 + l16) * pitch + k0 + 4 * lq;
    return cat(ld4(p), ld4(p + 16));
}
// A fragment from [k][m] storage (or a B fragment from [k][n] storage), by
// transposing reads: lane i of a 16-lane group receives column col0 + i.
__device__ __forceinline__ bf16x8 frag_cols(const uint16_t *M, int pitch, int col0, int k0, int l16, int lq) {
    const uint16_t *p = M + (k0 + 4 * lq + (l16 >> 2)) * pitch + col0 + 4 * (l16 & 3);
    return cat(ld4_tr(p), ld4_tr(p + 16 * pitch));
}
// The same from storage whose columns are key-permuted (kpos): every 4-column
// group stays contiguous, so each lane reads the same 8 bytes at their new place.
__device__ __forceinline__ bf16x8 frag_cols_kp(const uint16_t *M, int pitch, int col0, int k0, int l16, int lq) {
    const uint16_t *p = M + (k0 + 4 * lq + (l16 >> 2)) * pitch + kpos(col0 + 4 * (l16 & 3));
    return cat(ld4_tr(p), ld4_tr(p + 16 * pitch));
}
__device__ __forceinline__ float bf16_to_f(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }
// Rows row0 + 4 lq + r (r = 0..3) of column col0 + l16, as floats: a lane's
// C-tile positions, by one transposing read.
__device__ __forceinline__ f32x4 col4(const uint16_t *M, int pitch, int row0, int col0, int l16, int lq) {
    return up4(ld4_tr(M + (row0 + 4 * lq + (l16 >> 2)) * pitch + col0 + 4 * (l16 & 3)));
}

// Sum over each 16-lane row of the wave, left in the row's last lane.
__device__ __forceinline__ float row_sum16(float x) {
    x = dpp_add<0x111, 0xF>(x);
    x = dpp_add<0x112, 0xF>(x);
    x = dpp_add<0x114, 0xF>(x);
    x = dpp_add<0x118, 0xF>(x);
    return x;
}
__device__ __forceinline__ float lane63(float x) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void *p, int64_t i, float v) {
    if constexpr (BF16) reinterpret_cast<uint16_t *>(p)[i] = bf16_bits(v);
    else reinterpret_cast<float *>(p)[i] = v;
}
// four consecutive elements from element i (a multiple of 4)
template <bool BF16>
__device__ __forceinline__ void store_four(void *p, int64_t i, f32x4 v) {
    if constexpr (BF16) *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint16_t *>(p) + i) = cvt4(v);
    else *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p) + i) = v;
}

// The same rows into registers, 16 bytes of bf16 per piece, through a buffer
// resource that ends at the last row (rows from len on read as zero).
template <int D, bool BF16, int NP, int NT>
__device__ __forceinline__ void fetch_rows(v4u32 (&dst)[NP], const void *src, int64_t t0, int len, int heads,
                                           int head, int tid) {
    constexpr int PR = D / 8, ES = BF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(
        reinterpret_cast<const unsigned char *>(src) + ((t0 * heads + head) * D) * ES,
        static_cast<uint32_t>(len * heads * D * ES));
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int i = tid + j * NT, row = i / PR, col = 8 * (i % PR);
        dst[j] = __builtin_bit_cast(v4u32, buf_load8<BF16>(r, static_cast<uint32_t>((row * heads * D + col) * ES)));
    }
}

// Rows t0 .. t0+len-1 of a [tokens, heads, D] tensor (one head) into LDS
// [64][pitch] bf16 (rows from len on are zero): every load is issued before
// the first store.
template <int D, bool BF16, int NT>
__device__ __forceinline__ void stage_rows(uint16_t *dst, int pitch, const void *src, int64_t t0, int len,
                                           int heads, int head, int tid) {
    constexpr int PR = D / 8, NP = C * PR / NT;
    v4u32 r[NP];
    fetch_rows<D, BF16, NP, NT>(r, src, t0, len, heads, head, tid);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int i = tid + j * NT;
        *reinterpret_cast<v4u32 *>(dst + (i / PR) * pitch + 8 * (i % PR)) = r[j];
    }
}
// 16 bytes to / from LDS at p: one access where p is 16-byte aligned (A16),
// else two 8-byte ones.
template <bool A16>
__device__ __forceinline__ void st16(uint16_t *p, v4u32 v) {
    if constexpr (A16) {
        *reinterpret_cast<v4u32 *>(p) = v;
    } else {
        reinterpret_cast<v2u32 *>(p)[0] = v2u32{v[0], v[1]};
        reinterpret_cast<v2u32 *>(p)[1] = v2u32{v[2], v[3]};
    }
}
template <bool A16>
__device__ __forceinline__ v4u32 ld16(const uint16_t *p) {
    if constexpr (A16) {
        return *reinterpret_cast<const v4u32 *>(p);
    } else {
        const v2u32 x = reinterpret_cast<const v2u32 *>(p)[0], y = reinterpret_cast<const v2u32 *>(p)[1];
        return v4u32{x[0], x[1], y[0], y[1]};
    }
}
// Two such row blocks (of different tensors), all loads first; rows of P0
// and P1 elements.
template <int D, bool BF16, int NT, int P0, int P1>
__device__ __forceinline__ void stage_rows2(uint16_t *d0, const void *s0, int heads0, int head0, uint16_t *d1,
                                            const void *s1, int heads1, int head1, int64_t t0, int len, int tid) {
    constexpr int PR = D / 8, NP = C * PR / NT;
    v4u32 r0[NP], r1[NP];
    fetch_rows<D, BF16, NP, NT>(r0, s0, t0, len, heads0, head0, tid);
    fetch_rows<D, BF16, NP, NT>(r1, s1, t0, len, heads1, head1, tid);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int i = tid + j * NT, row = i / PR, col = 8 * (i % PR);
        st16<P0 % 8 == 0>(d0 + row * P0 + col, r0[j]);
        st16<P1 % 8 == 0>(d1 + row * P1 + col, r1[j]);
    }
}

// NP consecutive 16-byte pieces per thread of a contiguous block, strided by NT threads.
template <int NP, int NT>
__device__ __forceinline__ void fetch_block(v4u32 (&dst)[NP], const uint16_t *src, int tid) {
#pragma unroll
    for (int j = 0; j < NP; ++j) dst[j] = *reinterpret_cast<const v4u32 *>(src + 8 * (tid + j * NT));
}
// Which sequence and chunk a chunk row belongs to.
struct ChunkAt {
    int64_t n, c, t0;
    int len;
};
__device__ __forceinline__ bool chunk_at(const BwdArgs &a, int64_t r, ChunkAt &p) {
    int64_t bos, eos;
    if (a.map) {
        const int32_t n = a.map[2 * r];
        if (n < 0 || n >= a.n_seq) return false;
        p.n = n;
        p.c = a.map[2 * r + 1];
        bos = a.cu[n];
        eos = a.cu[n + 1];
    } else {
        const int64_t per = (a.seq_len + C - 1) / C;
        p.n = r / per;
        p.c = r % per;
        if (p.n >= a.n_seq) return false;
        bos = p.n * a.seq_len;
        eos = bos + a.seq_len;
    }
    bos = bos < 0 ? 0 : bos;
    eos = eos > a.total_tokens ? a.total_tokens : eos;
    p.t0 = bos + C * p.c;
    const int64_t len = eos - p.t0 < C ? eos - p.t0 : C;
    if (len <= 0) return false;
    p.len = static_cast<int>(len);
    return true;
}

// Raw bits of the gate of token t0 + lane, v-head h (zero past len): one
// buffer load, no branch; gate_value converts them.
template <bool GATE_BF16>
__device__ __forceinline__ uint32_t gate_bits(const void *g, int64_t t0, int len, int hv, int h, int lane) {
    constexpr int ES = GATE_BF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(reinterpret_cast<const unsigned char *>(g) + (t0 * hv + h) * ES,
                                                static_cast<uint32_t>(len * hv * ES));
    if constexpr (GATE_BF16) return static_cast<uint32_t>(buf_load<2>(r, static_cast<uint32_t>(lane * hv * ES)));
    else return buf_load<4>(r, static_cast<uint32_t>(lane * hv * ES));
}
template <bool GATE_BF16>
__device__ __forceinline__ float gate_value(uint32_t bits) {
    return __uint_as_float(GATE_BF16 ? bits << 16 : bits);
}

// Gate vectors of one chunk from the raw bits of its gate and beta, one token
// per lane of the calling wave: G log2(e) (chunk-local inclusive prefix sum),
// beta, and G_L log2(e).  The bits are loaded ahead (gate_bits) with the other
// loads of a phase, so that the scan does not wait for a load of its own.
template <bool GATE_BF16>
__device__ __forceinline__ void chunk_gates(uint32_t gbits, uint32_t bbits, float &G2, float &bv, float &GL2) {
    bv = gate_value<GATE_BF16>(bbits);
    G2 = wave_inclusive_scan(gate_value<GATE_BF16>(gbits) * kLog2e);
    GL2 = lane63(G2);
}

// --------------------------------------------------------------------------
// Per (chunk, NH v-heads of one q/k head): T.  With NH = 2 the k rows and
// K K^T are shared by the two v-heads, and all 8 waves work in the
// substitution phases (four per v-head).
// --------------------------------------------------------------------------
template <int D, int NH>
struct PrepLds {
    // Row pitches (bf16 elements) by how each array is read, against the 32
    // four-byte LDS banks: 8-byte row fragments (16 lanes, one row each) are
    // conflict-free at 2 mod 32 banks, transposing reads (4 rows of 32 bytes
    // per 16 lanes) at 8 mod 32; k, read both ways, takes 4 mod 32 (2-way).
    static constexpr int PK = D + 4;    // k [64][D]: row fragments
    static constexpr int PP = C + 4;    // A [64][64]: row fragments
    static constexpr int PD = 20;       // [16][16] bf16 blocks
    static constexpr int oK = 0;
    static constexpr int oA = oK + C * PK * 2;         // per v-head: diag(b) A~, strictly lower, [i][j]
    static constexpr int oG = oA + NH * C * PP * 2;    // per v-head f32 [64] x2: G log2(e), b
    static constexpr int oDi = oG + NH * 2 * C * 4;    // per v-head: bf16 inverses of the diagonal blocks of I + diag(b) A~
    static constexpr int bytes = oDi + NH * 4 * 16 * PD * 2;
};

template <int D, bool IN_BF16, bool GATE_BF16, int NH>
__global__ void __launch_bounds__(kBwdThreads) gdr_bwd_prep_kernel(BwdArgs a) {
    using Ly = PrepLds<D, NH>;
    constexpr int PK = Ly::PK, PP = Ly::PP, PD = Ly::PD;
    extern __shared__ __align__(16) unsigned char lds[];
    uint16_t *sK = reinterpret_cast<uint16_t *>(lds + Ly::oK);
    // per v-head s of the block: A at sA0 + s C PP, G log2(e) at sG0 + 2 s C
    // (b C further on), inverses at sDi0 + 64 s PD
    uint16_t *sA0 = reinterpret_cast<uint16_t *>(lds + Ly::oA);
    uint16_t *sDi0 = reinterpret_cast<uint16_t *>(lds + Ly::oDi);
    float *sG0 = reinterpret_cast<float *>(lds + Ly::oG);

    ChunkAt p;
    // one work item per (chunk row, group of NH v-heads); groups of one q/k
    // head share an L2
    const int ng = a.hv / NH;
    const int64_t item = gqa_xcd_item(blockIdx.x, gridDim.x, ng, a.hk);
    const int64_t crow = item / ng;
    if (!chunk_at(a, crow, p)) return;
    const int hb = static_cast<int>(item % ng) * NH;   // the block's first v-head
    const int hk = hb / (a.hv / a.hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, lq = lane >> 4;

    uint32_t gbits = 0u, bbits = 0u;
    if (wave < NH) {   // wave s: gate and beta of v-head hb + s
        gbits = gate_bits<GATE_BF16>(a.g, p.t0, p.len, a.hv, hb + wave, lane);
        bbits = gate_bits<GATE_BF16>(a.beta, p.t0, p.len, a.hv, hb + wave, lane);
    }
    {
        constexpr int PR = D / 8, NP = C * PR / kBwdThreads;
        v4u32 rk[NP];
        fetch_rows<D, IN_BF16, NP, kBwdThreads>(rk, a.k, p.t0, p.len, a.hk, hk, tid);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int i = tid + j * kBwdThreads;
            st16<PK % 8 == 0>(sK + (i / PR) * PK + 8 * (i % PR), rk[j]);
        }
    }
    for (int i = tid; i < NH * C * PP / 8; i += kBwdThreads)   // A: blocks above the diagonal stay zero
        reinterpret_cast<uint4 *>(sA0)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (wave < NH) {
        float G2, bv, GL2;
        chunk_gates<GATE_BF16>(gbits, bbits, G2, bv, GL2);
        sG0[2 * wave * C + lane] = G2;
        sG0[(2 * wave + 1) * C + lane] = bv;
    }
    __syncthreads();

    // K K^T, strictly lower, gated and times b per v-head (A): its ten lower
    // 16x16 blocks.  Formed transposed (the row block as the B operand), so
    // that a lane holds four consecutive columns j of one row i.
    for (int t = wave; t < 10; t += 8) {
        const int bi = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
        const int bj = t - bi * (bi + 1) / 2;
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32)
            acc = mfma32(frag_rows(sK, PK, 16 * bj, k0, l16, lq), frag_rows(sK, PK, 16 * bi, k0, l16, lq), acc);
        const int i = 16 * bi + l16, j0 = 16 * bj + 4 * lq;
#pragma unroll
        for (int s = 0; s < NH; ++s) {
            const float *sG2 = sG0 + 2 * s * C, *sB = sG2 + C;
            const float gi = sG2[i], bi_ = sB[i];
            f32x4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = fast_exp2(gi - sG2[j0 + r]);   // used only where j < i (exponent <= 0)
                out[r] = j0 + r < i ? bi_ * e * acc[r] : 0.f;
            }
            st4(sA0 + s * C * PP + i * PP + j0, cvt4(out));
        }
    }
    __syncthreads();

    // Diagonal blocks: column l16 of (I + A_bb)^-1 by forward substitution in
    // fp32 on the bf16 block (every 16-lane row of the wave computes the same
    // column).  Wave 4 s + b: block b of v-head s.
    const int s = wave >> 2;
    const uint16_t *sA = sA0 + s * C * PP;
    uint16_t *sDi = sDi0 + s * 64 * PD;
    f32x4 dcol = zero4();
    if (wave < 4 * NH) {
        const int b = wave & 3;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float sm = i == l16 ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) sm -= bf16_to_f(sA[(16 * b + i) * PP + 16 * b + m]) * x[m];
            x[i] = sm;
        }
        if (lq == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sDi[(16 * b + i) * PD + l16] = bf16_bits(x[i]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) dcol[r] = lq == 0 ? x[r] : lq == 1 ? x[4 + r] : lq == 2 ? x[8 + r] : x[12 + r];
    }
    __syncthreads();

    // Column block j of T: X_j = D_j, X_i = -D_i sum_{m=j}^{i-1} A_im X_m
    // (C tiles chained through registers).  T^T goes to memory.  Wave 4 s + j:
    // column block j of v-head s.
    if (wave < 4 * NH) {
        const int j = wave & 3;
        f32x4 X[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) X[i] = i == j ? dcol : zero4();
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            if (i > j) {
                f32x4 E = zero4();
#pragma unroll
                for (int m = 0; m < 3; ++m)
                    if (m >= j && m < i)
                        E = mfma16z(ld4(sA + (16 * i + l16) * PP + 16 * m + 4 * lq), cvt4(X[m]), E);
                X[i] = -mfma16z(ld4(sDi + (16 * i + l16) * PD + 4 * lq), cvt4(E), zero4());
            }
        }
        uint16_t *tg = a.tmat + (crow * a.hv + hb + s) * (C * C);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<bf16x4 *>(tg + (16 * j + l16) * C + 16 * i + 4 * lq) = cvt4(X[i]);
    }
}

// --------------------------------------------------------------------------
// Per (sequence, v-head), chunks in reverse order: the gradient of the state.
// Wave c owns dv columns [c*D/4, (c+1)*D/4) of dS' (fp32 C tiles, rows dk).
// --------------------------------------------------------------------------
template <int D>
struct ChainLds {
    // dO and T^T are read with transposing reads (pitch 8 mod 32 four-byte
    // banks: conflict-free); q both ways (4 mod 32: at most 2-way either
    // way); k with key-permuted columns (kpos): 16-byte row fragments in
    // C-tile key order, and transposing reads (2-way)
    static constexpr int PQ = D + 8;               // q
    static constexpr int PK = D + 16;              // dO
    static constexpr int PR = D + 16;              // k
    static constexpr int PT = C + 16;              // T^T
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + C * PQ * 2;
    static constexpr int oO = oK + C * PR * 2;
    static constexpr int oT = oO + C * PK * 2;     // T^T [64][PT]
    static constexpr int oG = oT + C * PT * 2;     // f32 [64] x4: scale e^G, e^{G_L - G}, G log2(e), b e^G; then e^{G_L}
    static constexpr int bytes = oG + 4 * C * 4 + 16;
};

template <int D, bool IN_BF16, bool GATE_BF16>
__global__ void __launch_bounds__(kChainThreads) gdr_bwd_chain_kernel(BwdArgs a) {
    using Ly = ChainLds<D>;
    constexpr int PQ = Ly::PQ, PK = Ly::PK, PKR = Ly::PR, PT = Ly::PT;
    constexpr int MT = D / 16;                        // dk tiles (and dv tiles)
    constexpr int NTW = D / 64;                       // dv tiles per wave
    constexpr int PR = D / 8;                         // 16-byte pieces per q / k / dO row
    constexpr int NQ = C * PR / kChainThreads;        // such pieces per thread
    constexpr int NT8 = C * (C / 8) / kChainThreads;  // 16-byte pieces of T^T per thread
    extern __shared__ __align__(16) unsigned char lds[];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(lds + Ly::oQ);
    uint16_t *sK = reinterpret_cast<uint16_t *>(lds + Ly::oK);
    uint16_t *sO = reinterpret_cast<uint16_t *>(lds + Ly::oO);
    uint16_t *sT = reinterpret_cast<uint16_t *>(lds + Ly::oT);
    float *sGs = reinterpret_cast<float *>(lds + Ly::oG);
    float *sLam = sGs + C;
    float *sG2 = sLam + C;
    float *sBG = sG2 + C;
    float *sGL = sBG + C;

    const int64_t item = gqa_xcd_item(blockIdx.x, gridDim.x, a.hv, a.hk);   // v-heads of a q/k head share an L2
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
    const int tid = threadIdx.x, wave = tid >> 6;
    const int colw = wave * (D / 4);
    const int64_t nch = (eos - bos + C - 1) / C;
    const int64_t off = a.offs ? static_cast<int64_t>(a.offs[n]) : n * ((a.seq_len + C - 1) / C);

    // Registers of the chunk being fetched while the previous one is processed:
    // rows of q, k and dO, T^T, this lane's gate and beta (wave 0; their raw
    // bits, by buffer loads that read zero past the segment end, converted at
    // use: a lane-dependent load or a conversion right after it would make
    // the wave wait there for every load of the prefetch).
    v4u32 pq[NQ], pk[NQ], po[NQ], pt[NT8];
    uint32_t pg = 0u, pb = 0u;
    // One quarter of the next chunk's loads (part 0: q rows, 1: k rows, 2: dO
    // rows, 3: T^T, the gate and beta).  The chain issues the quarters between the
    // phases of a chunk's products, so that the wave's vector-memory issue
    // overlaps its MFMA work instead of stalling ahead of it.
#define GDR_FETCH_PART(cc, part)                                                                       \
    {                                                                                                  \
        const int64_t t0_ = bos + C * (cc);                                                            \
        const int len_ = static_cast<int>(eos - t0_ < C ? eos - t0_ : C);                              \
        if ((part) == 0) fetch_rows<D, IN_BF16, NQ, kChainThreads>(pq, a.q, t0_, len_, a.hk, hk, tid); \
        if ((part) == 1) fetch_rows<D, IN_BF16, NQ, kChainThreads>(pk, a.k, t0_, len_, a.hk, hk, tid); \
        if ((part) == 2) fetch_rows<D, IN_BF16, NQ, kChainThreads>(po, a.dout, t0_, len_, a.hv, h, tid); \
        if ((part) == 3) {                                                                             \
            fetch_block<NT8, kChainThreads>(pt, a.tmat + ((off + (cc)) * a.hv + h) * (C * C), tid);     \
            if (wave == 0) {                                                                           \
                pg = gate_bits<GATE_BF16>(a.g, t0_, len_, a.hv, h, tid & 63);                          \
                pb = gate_bits<GATE_BF16>(a.beta, t0_, len_, a.hv, h, tid & 63);                       \
            }                                                                                          \
        }                                                                                              \
    }
#define GDR_FETCH(cc)                                                                                  \
    {                                                                                                  \
        GDR_FETCH_PART(cc, 0)                                                                          \
        GDR_FETCH_PART(cc, 1)                                                                          \
        GDR_FETCH_PART(cc, 2)                                                                          \
        GDR_FETCH_PART(cc, 3)                                                                          \
    }

    f32x4 dH[MT][NTW];
    {
        const int lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
        const float *src = a.dht ? a.dht + (n * a.hv + h) * D * D : nullptr;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dH[mt][nt][r] = src ? src[(16 * mt + 4 * lq + r) * D + colw + 16 * nt + l16] : 0.f;
    }
    GDR_FETCH(nch - 1)

    for (int64_t c = nch - 1; c >= 0; --c) {
        int lane = tid & 63;   // opaque per iteration: keeps per-lane addresses inside the loop
        asm volatile("" : "+v"(lane));
        const int l16 = lane & 15, lq = lane >> 4;
        const int64_t rh = (off + c) * a.hv + h;
        __syncthreads();   // the previous chunk's reads of LDS are done
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int i = tid + j * kChainThreads, row = i / PR, col = 8 * (i % PR);
            *reinterpret_cast<v4u32 *>(sQ + row * PQ + col) = pq[j];
            *reinterpret_cast<v2u32 *>(sK + row * PKR + kpos(col)) = v2u32{pk[j][0], pk[j][1]};
            *reinterpret_cast<v2u32 *>(sK + row * PKR + kpos(col + 4)) = v2u32{pk[j][2], pk[j][3]};
            *reinterpret_cast<v4u32 *>(sO + row * PK + col) = po[j];
        }
#pragma unroll
        for (int j = 0; j < NT8; ++j) {
            const int i = tid + j * kChainThreads;
            *reinterpret_cast<v4u32 *>(sT + (i / (C / 8)) * PT + 8 * (i % (C / 8))) = pt[j];
        }
        if (wave == 0) {
            const float G2 = wave_inclusive_scan(gate_value<GATE_BF16>(pg) * kLog2e);
            const float GL2 = lane63(G2);
            sGs[lane] = a.scale * fast_exp2(G2);
            sLam[lane] = fast_exp2(GL2 - G2);
            sG2[lane] = G2;
            sBG[lane] = gate_value<GATE_BF16>(pb) * fast_exp2(G2);
            if (lane == 0) sGL[0] = fast_exp2(GL2);
        }
        __syncthreads();

        // dU0 = (scale M o Q K^T)^T dO, this wave's dv columns.  Tile (ib, jb)
        // of P = scale M o Q K^T comes out of the MFMA in C layout (rows
        // 16 ib + 4 lq + r, column 16 jb + l16), which is the A-operand layout
        // of rows 16 jb + l16 of P^T at keys 16 ib + 4 lq + r: every wave
        // forms the lower tiles it needs in registers (measured faster than
        // sharing the ten tiles through LDS, which costs a barrier).
        // Row block ib of Q is read once and meets the k blocks jb <= ib; the
        // quarters of the next chunk's loads go out between the row blocks.
        f32x4 U0[4][NTW];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) U0[jb][nt] = zero4();
        float gjv[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) gjv[jb] = sG2[16 * jb + l16];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x4 half[2][4];   // P tiles (2 kk + hh, jb) in bf16; zero above the diagonal
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ib = 2 * kk + hh;
                if (c > 0) GDR_FETCH_PART(c - 1, ib)   // in flight during this chunk's products
                bf16x8 aq[D / 32];
#pragma unroll
                for (int k0 = 0; k0 < D; k0 += 32) aq[k0 / 32] = frag_rows(sQ, PQ, 16 * ib, k0, l16, lq);
                const f32x4 gi = *reinterpret_cast<const f32x4 *>(sG2 + 16 * ib + 4 * lq);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    if (jb > ib) {
                        half[hh][jb] = cvt4(zero4());
                        continue;
                    }
                    f32x4 sc = zero4();
#pragma unroll
                    for (int k0 = 0; k0 < D; k0 += 32)
                        sc = mfma32(aq[k0 / 32], kfrag8(sK, PKR, 16 * jb, k0, l16, lq), sc);
                    f32x4 pv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool keep = ib > jb || l16 <= 4 * lq + r;
                        pv[r] = keep ? a.scale * fast_exp2(gi[r] - gjv[jb]) * sc[r] : 0.f;
                    }
                    half[hh][jb] = cvt4(pv);
                }
            }
#pragma unroll
            for (int jb = 0; jb <= 2 * kk + 1; ++jb) {
                const bf16x8 af = cat(half[0][jb], half[1][jb]);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    U0[jb][nt] = mfma32(af, frag_cols(sO, PK, colw + 16 * nt, 32 * kk, l16, lq), U0[jb][nt]);
            }
        }

        // X1 = K dS', and dS' of this chunk stored for the per-chunk gradient
        // kernel from the same bf16 tiles (tile order: a lane's four values of
        // tile (mt, nt) as one 8-byte piece), the stores between the products
        f32x4 X1[4][NTW];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) X1[mt][nt] = zero4();
        uint16_t *dst = a.dhe + rh * D * D + (wave * MT * NTW * 64 + lane) * 4;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            bf16x8 bh[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const bf16x4 lo = cvt4(dH[2 * kk][nt]), hi = cvt4(dH[2 * kk + 1][nt]);
                *reinterpret_cast<bf16x4 *>(dst + (2 * kk * NTW + nt) * 64 * 4) = lo;
                *reinterpret_cast<bf16x4 *>(dst + ((2 * kk + 1) * NTW + nt) * 64 * 4) = hi;
                bh[nt] = cat(lo, hi);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 af = kfrag8(sK, PKR, 16 * mt, 32 * kk, l16, lq);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) X1[mt][nt] = mfma32(af, bh[nt], X1[mt][nt]);
            }
        }

        // dU = dU0 + diag(e^{G_L - G}) X1, stored in bf16 (the same tiling)
        uint16_t *ug = a.du + rh * (C * D);
        bf16x4 dUb[4][NTW];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                f32x4 u = U0[mt][nt];
#pragma unroll
                for (int r = 0; r < 4; ++r) u[r] += sLam[16 * mt + 4 * lq + r] * X1[mt][nt][r];
                dUb[mt][nt] = cvt4(u);
                *reinterpret_cast<bf16x4 *>(ug + ((mt * MT + colw / 16 + nt) * 64 + lane) * 4) = dUb[mt][nt];
            }

        // dS <- e^{G_L} dS' + Q^T diag(scale e^G) dO - w^T dU, with
        // w = T diag(b e^G) K formed here: tile (tb, db) of w comes out of the
        // MFMA in C layout (rows 16 tb + 4 lq + r, column 16 db + l16), the
        // A-operand layout of rows 16 db + l16 of w^T at keys 16 tb + 4 lq + r.
        // Its A operand, rows of T diag(b e^G), is read transposed from T^T
        // with each key scaled by its b e^G; T is lower triangular, so row
        // blocks 0-1 need keys 0-31 only.
        const float gl = sGL[0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) dH[mt][nt] = dH[mt][nt] * gl;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 bo[NTW], bu[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                bf16x8 f = frag_cols(sO, PK, colw + 16 * nt, 32 * kk, l16, lq);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float x = static_cast<float>(f[s]);
                    f[s] = static_cast<__bf16>(x * sGs[32 * kk + 16 * (s >> 2) + 4 * lq + (s & 3)]);
                }
                bo[nt] = f;
                bu[nt] = cat(neg4(dUb[2 * kk][nt]), neg4(dUb[2 * kk + 1][nt]));
            }
            bf16x8 at[2][2];   // [tb - 2 kk][key block kk2 <= kk]
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int kk2 = 0; kk2 <= kk; ++kk2) {
                    bf16x8 f = frag_cols(sT, PT, 16 * (2 * kk + hh), 32 * kk2, l16, lq);
                    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(sBG + 32 * kk2 + 4 * lq);
                    const f32x4 b1 = *reinterpret_cast<const f32x4 *>(sBG + 32 * kk2 + 16 + 4 * lq);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        f[e] = static_cast<__bf16>(static_cast<float>(f[e]) * (e < 4 ? b0[e] : b1[e - 4]));
                    at[hh][kk2] = f;
                }
            // the w tiles of dk block mt + 1 are formed while block mt's
            // products run, so their results are ready when converted
            auto wtiles = [&](int mt, f32x4 &w0, f32x4 &w1) __attribute__((always_inline)) {
                w0 = zero4();
                w1 = zero4();
#pragma unroll
                for (int kk2 = 0; kk2 <= kk; ++kk2) {
                    const bf16x8 bk = frag_cols_kp(sK, PKR, 16 * mt, 32 * kk2, l16, lq);
                    w0 = mfma32(at[0][kk2], bk, w0);
                    w1 = mfma32(at[1][kk2], bk, w1);
                }
            };
            f32x4 wn0, wn1;
            wtiles(0, wn0, wn1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 w0 = wn0, w1 = wn1;
                if (mt + 1 < MT) wtiles(mt + 1, wn0, wn1);
                const bf16x8 aq = frag_cols(sQ, PQ, 16 * mt, 32 * kk, l16, lq);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) dH[mt][nt] = mfma32(aq, bo[nt], dH[mt][nt]);
                const bf16x8 aw = cat(cvt4(w0), cvt4(w1));
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) dH[mt][nt] = mfma32(aw, bu[nt], dH[mt][nt]);
            }
        }
    }

    if (a.dh0) {
        const int lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
        float *dst = a.dh0 + (n * a.hv + h) * D * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(16 * mt + 4 * lq + r) * D + colw + 16 * nt + l16] = dH[mt][nt][r];
    }
#undef GDR_FETCH
#undef GDR_FETCH_PART
}

// --------------------------------------------------------------------------
// Per (chunk, q/k head), looping over the v-heads of the group: all input
// gradients of the chunk's tokens.
// --------------------------------------------------------------------------
// (dv, first dk) of 8-byte piece P (four dk rows of one dv column) of a bf16
// state in the forward kernel's tile order (4 chain waves of d/4 columns,
// tiles (kb, nt), kb < d/16, nt < d/64)
template <int D>
__device__ __forceinline__ void fwd_piece(int P, int &dv, int &dk0) {
    constexpr int NTW = D / 64, KB = D / 16;
    const int ln = P & 63, t = P >> 6, nt = t % NTW, kb = (t / NTW) % KB, w = t / (NTW * KB);
    dk0 = 32 * (kb >> 1) + 8 * (ln >> 4) + 4 * (kb & 1);
    dv = w * (D / 4) + 4 * NTW * ((ln & 15) >> 2) + 4 * nt + (ln & 3);
}
// The same for the chain kernel's tile order (tiles (mt, nt), mt < d/16, nt < d/64)
template <int D>
__device__ __forceinline__ void chain_piece(int P, int &dv, int &dk0) {
    constexpr int NTW = D / 64, MT = D / 16;
    const int ln = P & 63, t = P >> 6, nt = t % NTW, mt = (t / NTW) % MT, w = t / (NTW * MT);
    dk0 = 16 * mt + 4 * (ln >> 4);
    dv = w * (D / 4) + 16 * nt + (ln & 15);
}
// bf16 element e (0..3) of four packed in two words, as bits / as float
__device__ __forceinline__ uint32_t bf16_of(v2u32 x, int e) { return (e & 1) ? x[e >> 1] >> 16 : x[e >> 1] & 0xFFFFu; }

template <int D>
struct GradLds {
    // Row pitches (bf16 elements), chosen by timing the kernel over a sweep
    // of them (the results are bit-identical).  q and v, read by transposing
    // reads only: 16 mod 64
    static constexpr int PQ = D + 16;
    // k: 8-byte row fragments (X = K S) and transposing reads
    static constexpr int PK = D + 12;
    // dO, U, dW: key-permuted columns (kpos), read as 16-byte fragments
    // (16-byte aligned rows)
    static constexpr int PKP = D + 16;
    // S^T / dS'^T: row fragments, transposing reads, pieces of four rows
    static constexpr int PS = D + 12;
    // T^T and the Zs, dBn, dB tiles: 8-byte row fragments, transposing reads
    // and 8-byte stores (rows only 8-byte aligned)
    static constexpr int PP = C + 4;
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + C * PQ * 2;
    static constexpr int oO = oK + C * PK * 2;        // dO [64][PKP]
    static constexpr int oV = oO + C * PKP * 2;       // V [64][PQ]; later Zs, dBn, dB [64][PP] each
    static constexpr int oT = oV + C * PQ * 2;        // T^T [64][PP]
    static constexpr int szVT = (C * PQ * 2 + C * PP * 2) > 3 * C * PP * 2 ? (C * PQ * 2 + C * PP * 2) : 3 * C * PP * 2;
    static constexpr int oS = oV + szVT;              // S^T, later dS'^T: [dv][PS] (rows dv, columns dk)
    static constexpr int oU = oS + D * PS * 2;        // U [64][PKP]
    static constexpr int oW = oU + C * PKP * 2;       // dW [64][PKP]
    static constexpr int oG = oW + C * PKP * 2;        // f32 [64] x4: G log2(e), b, e^G, e^{G_L - G}
    static constexpr int oR = oG + 4 * C * 4;         // f32 [8][64] x2: per-wave row sums for dG and db
    static constexpr int oX = oR + 2 * 8 * C * 4;     // f32 [8] x2: per-wave sums of <dS', S> and the lambda k.(U dS'^T) terms; e^{G_L}
    static constexpr int bytes = oX + 2 * 8 * 4 + 16;
};

template <int D, bool IN_BF16, bool GATE_BF16>
__global__ void __launch_bounds__(kBwdThreads) gdr_bwd_grads_kernel(BwdArgs a) {
    using Ly = GradLds<D>;
    constexpr int PQ = Ly::PQ, PK = Ly::PK, PKP = Ly::PKP, PS = Ly::PS, PP = Ly::PP, NTD = D / 16;
    extern __shared__ __align__(16) unsigned char lds[];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(lds + Ly::oQ);
    uint16_t *sK = reinterpret_cast<uint16_t *>(lds + Ly::oK);
    uint16_t *sO = reinterpret_cast<uint16_t *>(lds + Ly::oO);
    uint16_t *sV = reinterpret_cast<uint16_t *>(lds + Ly::oV);
    uint16_t *sT = reinterpret_cast<uint16_t *>(lds + Ly::oT);
    uint16_t *sZs = reinterpret_cast<uint16_t *>(lds + Ly::oV);
    uint16_t *sBn = sZs + C * PP;
    uint16_t *sBb = sBn + C * PP;
    uint16_t *sS = reinterpret_cast<uint16_t *>(lds + Ly::oS);
    uint16_t *sU = reinterpret_cast<uint16_t *>(lds + Ly::oU);
    uint16_t *sDW = reinterpret_cast<uint16_t *>(lds + Ly::oW);
    float *sG2 = reinterpret_cast<float *>(lds + Ly::oG);
    float *sB = sG2 + C;
    float *sGam = sB + C;
    float *sLam = sGam + C;
    float *sRG = reinterpret_cast<float *>(lds + Ly::oR);
    float *sRB = sRG + 8 * C;
    float *sXd = reinterpret_cast<float *>(lds + Ly::oX);
    float *sXl = sXd + 8;
    float *sGL = sXl + 8;

    ChunkAt p;
    if (!chunk_at(a, blockIdx.x, p)) return;
    const int hk = blockIdx.y;
    const int G = a.hv / a.hk;
    const int tid = threadIdx.x, wave = tid >> 6;
    const bool colwave = wave < NTD;   // owns column tile `wave` in the column-split phases
    const int nt = wave;

    stage_rows2<D, IN_BF16, kBwdThreads, PQ, PK>(sQ, a.q, a.hk, hk, sK, a.k, a.hk, hk, p.t0, p.len, tid);

    f32x4 accQ[4], accK[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) accQ[mt] = accK[mt] = zero4();

    // dg: reverse prefix sums of dG within the chunk (wave 0); dbeta (wave 2);
    // for v-head hv_ of parity hp_, from the row sums its phases left in LDS.
    // Run at the next v-head's staging, while that one's loads are in flight;
    // meanwhile wave 1 forms the next v-head's gate vectors, so e^{G_L} is
    // kept per v-head parity (the value read here is not overwritten).
#define GDR_GRAD_DG(hv_, ln_, hp_)                                                             \
    if (wave == 0) {                                                                         \
        float dG = 0.f;                                                                      \
        for (int w = 0; w < NTD; ++w) dG += sRG[w * C + (ln_)];                              \
        if ((ln_) == 63) {                                                                   \
            float dot = 0.f, kl = 0.f;                                                       \
            for (int w = 0; w < 8; ++w) dot += sXd[w];                                       \
            for (int w = 0; w < NTD; ++w) kl += sXl[w];                                      \
            dG += sGL[(hp_)] * dot + kl;                                                     \
        }                                                                                    \
        const float inc = wave_inclusive_scan(dG);                                           \
        const float dgv = lane63(inc) - inc + dG;                                            \
        if ((ln_) < p.len) a.dg[(p.t0 + (ln_)) * a.hv + (hv_)] = dgv;                         \
    } else if (wave == 2) {                                                                  \
        float db = 0.f;                                                                      \
        for (int w = 0; w < NTD; ++w) db += sRB[w * C + (ln_)];                              \
        if ((ln_) < p.len) a.dbeta[(p.t0 + (ln_)) * a.hv + (hv_)] = db;                       \
    }
    for (int hh = 0; hh < G; ++hh) {
        // lane indices re-derived opaquely in every iteration, so that the
        // compiler does not hoist (and spill) per-lane addresses out of the loop
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        const int l16 = lane & 15, lq = lane >> 4;
        const int h = hk * G + hh;
        const int64_t rh = static_cast<int64_t>(blockIdx.x) * a.hv + h;
        // the state at the chunk start: bf16 after the previous chunk, else h0 (fp32) or zero
        const uint16_t *Sb = p.c > 0 ? a.hck + (rh - a.hv) * D * D : nullptr;
        const float *Sg = p.c == 0 && a.h0 ? a.h0 + (p.n * a.hv + h) * D * D : nullptr;
        bf16x4 ub[4];   // this wave's dU tiles (dv tile nt), bf16
        uint32_t gbits = 0u, bbits = 0u;   // wave 1: raw gate and beta bits of the chunk
        if (colwave) {
            const uint16_t *ug = a.du + rh * (C * D);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ub[mt] = *reinterpret_cast<const bf16x4 *>(ug + ((mt * NTD + nt) * 64 + lane) * 4);
        }
        {
            // all of this v-head's staging loads are issued before the barrier
            // (they go to registers), and so before the first store
            constexpr int PR = D / 8, NP = C * PR / kBwdThreads, NT8 = C * C / 8 / kBwdThreads;
            constexpr int NS4 = D * D / 4 / kBwdThreads;   // 8-byte pieces (4 bf16) of the state per thread
            v4u32 rv[NP], ro[NP], rt[NT8];
            v2u32 rs4[NS4];
            if (wave == 1) {
                gbits = gate_bits<GATE_BF16>(a.g, p.t0, p.len, a.hv, h, lane);
                bbits = gate_bits<GATE_BF16>(a.beta, p.t0, p.len, a.hv, h, lane);
            }
            fetch_rows<D, IN_BF16, NP, kBwdThreads>(rv, a.v, p.t0, p.len, a.hv, h, tid);
            fetch_rows<D, IN_BF16, NP, kBwdThreads>(ro, a.dout, p.t0, p.len, a.hv, h, tid);
            if (Sb) {
#pragma unroll
                for (int j = 0; j < NS4; ++j) rs4[j] = *reinterpret_cast<const v2u32 *>(Sb + 4 * (tid + j * kBwdThreads));
            } else {
                // a sequence's first chunk: h0 ([dk][dv] fp32) rounded to bf16
                // here (the only chunk whose staging waits for its state loads)
#pragma unroll
                for (int j = 0; j < NS4; ++j) {
                    const float *src = Sg ? Sg + 4 * (tid + j * kBwdThreads) : nullptr;
                    rs4[j] = __builtin_bit_cast(v2u32, cvt4(src ? *reinterpret_cast<const f32x4 *>(src) : zero4()));
                }
            }
            const uint16_t *tg = a.tmat + rh * (C * C);
#pragma unroll
            for (int j = 0; j < NT8; ++j) rt[j] = *reinterpret_cast<const v4u32 *>(tg + 8 * (tid + j * kBwdThreads));
            __syncthreads();   // the previous v-head's reads of LDS are done
            if (hh > 0) GDR_GRAD_DG(h - 1, lane, (hh - 1) & 1)   // the previous v-head's, while the loads fly
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int i = tid + j * kBwdThreads, off = (i / PR) * PQ + 8 * (i % PR);
                st16<PQ % 8 == 0>(sV + off, rv[j]);
                // dO with key-permuted columns: the piece's two halves of four
                const int orow = i / PR, oc = 8 * (i % PR);
                *reinterpret_cast<v2u32 *>(sO + orow * PKP + kpos(oc)) = v2u32{ro[j][0], ro[j][1]};
                *reinterpret_cast<v2u32 *>(sO + orow * PKP + kpos(oc + 4)) = v2u32{ro[j][2], ro[j][3]};
            }
            // S^T [dv][dk] in LDS: the bf16 state piece by piece (four dk of
            // one dv: one 8-byte store), h0 element by element.  Elements are
            // taken with integer shifts (extracting __bf16 vector elements for
            // 2-byte stores has been compiled to stores of one register for all)
            if (Sb) {
#pragma unroll
                for (int j = 0; j < NS4; ++j) {
                    int dvp, dk0;
                    fwd_piece<D>(tid + j * kBwdThreads, dvp, dk0);
                    *reinterpret_cast<v2u32 *>(sS + dvp * PS + dk0) = rs4[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < NS4; ++j) {
                    const int i = 4 * (tid + j * kBwdThreads), dk = i / D, dv0 = i % D;
#pragma unroll
                    for (int e = 0; e < 4; ++e) sS[(dv0 + e) * PS + dk] = static_cast<uint16_t>(bf16_of(rs4[j], e));
                }
            }
#pragma unroll
            for (int j = 0; j < NT8; ++j) {
                const int i = tid + j * kBwdThreads;
                st16<PP % 8 == 0>(sT + (i / (C / 8)) * PP + 8 * (i % (C / 8)), rt[j]);
            }
        }
        if (wave == 1) {
            float G2, bv, GL2;
            chunk_gates<GATE_BF16>(gbits, bbits, G2, bv, GL2);
            sG2[lane] = G2;
            sB[lane] = bv;
            sGam[lane] = fast_exp2(G2);
            sLam[lane] = fast_exp2(GL2 - G2);
            if (lane == 0) sGL[hh & 1] = fast_exp2(GL2);
        }
        __syncthreads();

        // X = K S, R~ = V - e^G X, U = T diag(b) R~, dW = T^T dU, dV = b dW (dv tile nt).
        // U and dW are also formed transposed (the same products with the
        // operands swapped: a lane then holds four consecutive dv columns of
        // one token), for 8-byte stores of U, dW and dV.
        if (colwave) {
            f32x4 Rt[4], Ut[4], dW[4], dWt[4];
            bf16x4 wb[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Rt[mt] = zero4();
            for (int kk = 0; kk < D / 32; ++kk) {
                const bf16x8 bs = frag_rows(sS, PS, 16 * nt, 32 * kk, l16, lq);   // S^T rows: B = S [dk][dv]
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) Rt[mt] = mfma32(frag_rows(sK, PK, 16 * mt, 32 * kk, l16, lq), bs, Rt[mt]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 w;
                const f32x4 vv = col4(sV, PQ, 16 * mt, 16 * nt, l16, lq);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * mt + 4 * lq + r;
                    Rt[mt][r] = vv[r] - sGam[i] * Rt[mt][r];   // R~ = V - e^G X
                    w[r] = sB[i] * Rt[mt][r];
                }
                wb[mt] = cvt4(w);
                Ut[mt] = dW[mt] = dWt[mt] = zero4();
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 bw = cat(wb[2 * kk], wb[2 * kk + 1]);
                const bf16x8 bu = cat(ub[2 * kk], ub[2 * kk + 1]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const bf16x8 tr = frag_rows(sT, PP, 16 * mt, 32 * kk, l16, lq);
                    Ut[mt] = mfma32(bw, frag_cols(sT, PP, 16 * mt, 32 * kk, l16, lq), Ut[mt]);
                    dW[mt] = mfma32(tr, bu, dW[mt]);
                    dWt[mt] = mfma32(bu, tr, dWt[mt]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int i = 16 * mt + l16, c = 16 * nt + 4 * lq;   // transposed tiles: token i, dv c..c+3
                const float bi = sB[i];
                if (i < p.len) store_four<IN_BF16>(a.dv, ((p.t0 + i) * a.hv + h) * D + c, f32x4{bi * dWt[mt][0], bi * dWt[mt][1], bi * dWt[mt][2], bi * dWt[mt][3]});
                st4(sU + i * PKP + kpos(c), cvt4(Ut[mt]));
                st4(sDW + i * PKP + kpos(c), cvt4(dWt[mt]));
                float pb[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) pb[r] = row_sum16(dW[mt][r] * Rt[mt][r]);
                if (l16 == 15) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sRB[wave * C + 16 * mt + 4 * lq + r] = pb[r];
                }
            }
        }
        __syncthreads();

        // dQ1 = dO S^T, dK1 = dW S^T (dk tile nt)
        constexpr int NDS = D * D / 4 / kBwdThreads;   // 8-byte pieces of dS' per thread
        v2u32 pds[NDS];
#pragma unroll
        for (int j = 0; j < NDS; ++j) pds[j] = *reinterpret_cast<const v2u32 *>(a.dhe + rh * D * D + 4 * (tid + j * kBwdThreads));
        f32x4 dQt[4], dK1[4];   // dQt: scale e^G dO S^T, then + Zs K
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dQt[mt] = dK1[mt] = zero4();
        if (colwave) {
            for (int kk = 0; kk < D / 32; ++kk) {
                const bf16x8 bs = frag_cols(sS, PS, 16 * nt, 32 * kk, l16, lq);   // B = S^T
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    dQt[mt] = mfma32(kfrag8(sO, PKP, 16 * mt, 32 * kk, l16, lq), bs, dQt[mt]);
                    dK1[mt] = mfma32(kfrag8(sDW, PKP, 16 * mt, 32 * kk, l16, lq), bs, dK1[mt]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) dQt[mt][r] *= a.scale * sGam[16 * mt + 4 * lq + r];
        }
        __syncthreads();   // S, V and T are no longer read

        // dS' into LDS over S, with <dS', S> taken on the way; Zs, dBn, dB
        {
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < NDS; ++j) {
                int dvp, dk0;
                chain_piece<D>(tid + j * kBwdThreads, dvp, dk0);
                v2u32 *sp = reinterpret_cast<v2u32 *>(sS + dvp * PS + dk0);
                const v2u32 sv = *sp;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    part += __uint_as_float(bf16_of(pds[j], e) << 16) * __uint_as_float(bf16_of(sv, e) << 16);
                *sp = pds[j];
            }
            part = lane63(wave_inclusive_scan(part));
            if (lane == 0) sXd[wave] = part;
        }
        // tiles (bi, bj) in the order of a list with the ten lower tiles
        // (bi >= bj) first, so that the two waves of each SIMD share about
        // the same number of them; the six upper tiles only store zeros
        for (int t = wave; t < 16; t += 8) {
            constexpr uint64_t kTiles = 0x2110003333222110ull;   // bi of list entry t in nibble t ...
            constexpr uint64_t kTilesJ = 0x3323213210210100ull;  // ... and bj
            const int bi = static_cast<int>((kTiles >> (4 * t)) & 15), bj = static_cast<int>((kTilesJ >> (4 * t)) & 15);
            f32x4 z0 = zero4(), z1 = zero4();
            // transposed tiles (U rows as the A operand): a lane holds four
            // consecutive columns j of one row i, for 8-byte stores
            if (bi >= bj) {
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk) {
                    const bf16x8 bu = kfrag8(sU, PKP, 16 * bj, 32 * kk, l16, lq);
                    z0 = mfma32(bu, kfrag8(sO, PKP, 16 * bi, 32 * kk, l16, lq), z0);
                    z1 = mfma32(bu, kfrag8(sDW, PKP, 16 * bi, 32 * kk, l16, lq), z1);
                }
            }
            const int i = 16 * bi + l16, j0 = 16 * bj + 4 * lq;
            const float gi = sG2[i], bti = sB[i];
            f32x4 zs, bn, bb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = j0 + r;
                const float e = fast_exp2(gi - sG2[j]);   // used only where j <= i
                zs[r] = j <= i ? a.scale * e * z0[r] : 0.f;
                bn[r] = j < i ? -e * z1[r] : 0.f;
                bb[r] = bti * bn[r];
            }
            st4(sZs + i * PP + j0, cvt4(zs));
            st4(sBn + i * PP + j0, cvt4(bn));
            st4(sBb + i * PP + j0, cvt4(bb));
        }
        __syncthreads();

        // dK5 = U dS'^T, Zs K, dBn K, Zs^T Q, dB^T K (dk tile nt); combine
        if (colwave) {
            // Kc: the column uses of k, lambda (U dS'^T) + Zs^T Q + dB^T K
            f32x4 Kc[4], Yb[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Kc[mt] = Yb[mt] = zero4();
            for (int kk = 0; kk < D / 32; ++kk) {
                const bf16x8 bd = frag_cols(sS, PS, 16 * nt, 32 * kk, l16, lq);   // B = dS'^T
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) Kc[mt] = mfma32(kfrag8(sU, PKP, 16 * mt, 32 * kk, l16, lq), bd, Kc[mt]);
            }
            float lastp = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const f32x4 kv = col4(sK, PK, 16 * mt, 16 * nt, l16, lq);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * mt + 4 * lq + r;
                    Kc[mt][r] *= sLam[i];
                    lastp += kv[r] * Kc[mt][r];
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 bk = frag_cols(sK, PK, 16 * nt, 32 * kk, l16, lq);
                const bf16x8 bq = frag_cols(sQ, PQ, 16 * nt, 32 * kk, l16, lq);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    dQt[mt] = mfma32(frag_rows(sZs, PP, 16 * mt, 32 * kk, l16, lq), bk, dQt[mt]);
                    Yb[mt] = mfma32(frag_rows(sBn, PP, 16 * mt, 32 * kk, l16, lq), bk, Yb[mt]);
                    Kc[mt] = mfma32(frag_cols(sZs, PP, 16 * mt, 32 * kk, l16, lq), bq, Kc[mt]);
                    Kc[mt] = mfma32(frag_cols(sBb, PP, 16 * mt, 32 * kk, l16, lq), bk, Kc[mt]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                float pg[4], pb[4];
                const f32x4 q4 = col4(sQ, PQ, 16 * mt, 16 * nt, l16, lq), k4 = col4(sK, PK, 16 * mt, 16 * nt, l16, lq);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * mt + 4 * lq + r;
                    const float qv = q4[r], kv = k4[r];
                    const float bt = sB[i];
                    const float dq = dQt[mt][r];
                    const float dkr = bt * (Yb[mt][r] - sGam[i] * dK1[mt][r]);
                    const float dkc = Kc[mt][r];
                    accQ[mt][r] += dq;
                    accK[mt][r] += dkr + dkc;
                    pg[r] = row_sum16(qv * dq + kv * (dkr - dkc));
                    pb[r] = row_sum16(kv * Yb[mt][r]);
                }
                if (l16 == 15) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * mt + 4 * lq + r;
                        sRG[wave * C + i] = pg[r];
                        sRB[wave * C + i] += pb[r];
                    }
                }
            }
            lastp = lane63(wave_inclusive_scan(lastp));
            if (lane == 0) sXl[wave] = lastp;
        }
    }
    // the last v-head's dg and dbeta
    __syncthreads();
    GDR_GRAD_DG(hk * G + G - 1, tid & 63, (G - 1) & 1)
#undef GDR_GRAD_DG

    // dq, dk summed over the v-heads of this q/k head
    const int lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
    if (colwave) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * lq + r;
                if (i < p.len) {
                    const int64_t o = ((p.t0 + i) * a.hk + hk) * D + 16 * nt + l16;
                    store_elem<IN_BF16>(a.dq, o, accQ[mt][r]);
                    store_elem<IN_BF16>(a.dk, o, accK[mt][r]);
                }
            }
    }
}

template <typename K>
hipError_t launch_with_lds(K kern, dim3 grid, dim3 block, int lds, hipStream_t stream, const BwdArgs &a) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, lds, stream, a);
    return hipGetLastError();
}

template <int D, bool IN_BF16, bool GATE_BF16>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
    const unsigned rows = static_cast<unsigned>(a.rows);
    // two v-heads per prep block where they share a q/k head
    hipError_t e = (a.hv / a.hk) % 2 == 0
                       ? launch_with_lds(gdr_bwd_prep_kernel<D, IN_BF16, GATE_BF16, 2>,
                                         dim3(static_cast<unsigned>(rows * (a.hv / 2))), dim3(kBwdThreads),
                                         PrepLds<D, 2>::bytes, stream, a)
                       : launch_with_lds(gdr_bwd_prep_kernel<D, IN_BF16, GATE_BF16, 1>,
                                         dim3(static_cast<unsigned>(rows * a.hv)), dim3(kBwdThreads),
                                         PrepLds<D, 1>::bytes, stream, a);
    if (e != hipSuccess) return e;
    e = launch_with_lds(gdr_bwd_chain_kernel<D, IN_BF16, GATE_BF16>,
                        dim3(static_cast<unsigned>(a.n_seq * a.hv)), dim3(kChainThreads),
                        ChainLds<D>::bytes, stream, a);
    if (e != hipSuccess) return e;
    return launch_with_lds(gdr_bwd_grads_kernel<D, IN_BF16, GATE_BF16>, dim3(rows, a.hk),
                           dim3(kBwdThreads), GradLds<D>::bytes, stream, a);
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t s) {
    if (a.in_bf16) return a.gate_bf16 ? launch_bwd_t<D, true, true>(a, s) : launch_bwd_t<D, true, false>(a, s);
    return a.gate_bf16 ? launch_bwd_t<D, false, true>(a, s) : launch_bwd_t<D, false, false>(a, s);
}

static_assert(GradLds<128>::bytes <= 160 * 1024, "gradient kernel LDS");
static_assert(PrepLds<128, 2>::bytes <= 160 * 1024, "prep kernel LDS");
static_assert(ChainLds<128>::bytes <= 160 * 1024, "chain kernel LDS");

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
    if (a.n_seq == 0 || a.hv == 0 || a.rows == 0) return hipSuccess;
    return a.d == 64 ? launch_bwd_d<64>(a, stream) : launch_bwd_d<128>(a, stream);
}

}  // namespace gdr
