// HIP kernel of the chunked gated delta rule with per-channel gates (the
// KDA-style variant of "feat(cake_kda): add paired recurrent training for
// SM100a and SM103a", whose raw gate carries one value per key channel), for
// gfx950.  The decay exp(g_t) becomes diag(exp(g_t)), g_t in R^dk, on the key
// side of the state:  S_t = S_{t-1} diag(e^{g_t}) (I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = scale S_t q_t.  g is taken as the log-decay itself (the transform that
// makes it from a raw gate is not defined on the pages).
//
// Chunk form.  With G the chunk-local prefix sums of g (per channel, rows past
// the segment end padded with g = b = 0), the exponentials are folded into the
// operands with one reference per 16-row block: R_b = G at the row before
// block b (R_0 = 0), b(i) the block of row i,
//
//   q~_i = q_i o e^{G_i - R_b(i)},  k~_i = k_i o e^{G_i - R_b(i)}       (<= 1)
//   k^(b)_j = k_j o e^{R_b - G_j}  for j < 16 (b + 1)      (<= 1 for j < 16 b)
//   A_ij = b_i k~_i . k^(b(i))_j (j < i),  P_ij = scale q~_i . k^(b(i))_j (j <= i)
//   U  = (I + A)^-1 diag(b) (V - (k o e^G) H)
//   O  = scale (q o e^G) H + P U
//   H <- diag(e^{G_L}) H + (k o e^{G_L - G})^T U
//
// Every factor is at most 1 except inside a diagonal block, where it is at
// most e^{-(the block's decay)}: a channel's log-decay summed over 16 tokens
// must stay above about -87 (fp32 and bf16 exponent range), i.e. about -5.4
// per token, which holds the pages' safe-gate lower bound of -5.  A block
// beyond it sets GDR_DEVSTAT_KDA_RANGE in the device status word.
//
// One work-group of 8 waves per (sequence, v-head) walks its chunks in order;
// wave w owns dv columns [16w, 16w + 16) of the fp32 state (MFMA C tiles, rows
// dk).  Per chunk: the gate scan (all threads: two adjacent channels and an
// eighth of the tokens each) and the gated operands into LDS; the ten lower blocks of A and
// of P (the four waves that make the diagonal blocks of A also invert them,
// 16x16 by fp32 substitution), then each wave's (k o e^G) H and (q o e^G) H
// (H taken from the wave's own state registers, whose C-tile layout is the B
// operand's); then per wave U by block forward substitution over its
// columns, O and the state update.
#include "gdr_internal.h"
#include "gdr_device.h"

#include <stdint.h>

#include <type_traits>

namespace gdr {
namespace {

constexpr int kKdaThreads = 512;

__device__ __forceinline__ bf16x8 kfrag_cols(const uint16_t *M, int pitch, int col0, int k0, int l16, int lq) {
    const uint16_t *p = M + (k0 + 4 * lq + (l16 >> 2)) * pitch + col0 + 4 * (l16 & 3);
    return cat(ld4_tr(p), ld4_tr(p + 16 * pitch));
}

template <bool BF16>
using VRaw = typename std::conditional<BF16, __bf16, float>::type;
// One element at byte offset off (the whole offset in the range-checked
// vector offset) of a buffer range, as loaded; past the range it reads 0.
template <bool BF16>
__device__ __forceinline__ VRaw<BF16> rd_raw(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BF16) return __builtin_bit_cast(__bf16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
    else return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// Two adjacent channels of one token, as loaded: bf16 pairs in one 32-bit
// word, f32 pairs in two.
template <bool BF16>
using PRaw = typename std::conditional<BF16, uint32_t, v2u32>::type;
template <bool BF16>
__device__ __forceinline__ PRaw<BF16> rd_pair(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BF16) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else return __builtin_bit_cast(v2u32, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <bool BF16>
__device__ __forceinline__ float pair_val(PRaw<BF16> x, int e) {
    if constexpr (BF16) return __uint_as_float(e ? (x & 0xffff0000u) : (x << 16));
    else return __uint_as_float(x[e]);
}
// Channels 2 cp, 2 cp + 1 of g, q and k for the TPG tokens of scan group grp,
// each pair as loaded (nothing is computed on them here, so the loads stay
// in flight), through ranges that end at the segment's end.
template <int D, int TPG, bool IN_BF16, bool GATE_BF16>
__device__ __forceinline__ void kda_fetch_gate(const FwdArgs &a, int64_t t0, int len, int h, int hk, int cp,
                                               int grp, PRaw<GATE_BF16> (&pg)[TPG], PRaw<IN_BF16> (&pq)[TPG],
                                               PRaw<IN_BF16> (&pk)[TPG]) {
    constexpr uint32_t ES = IN_BF16 ? 2 : 4, GS = GATE_BF16 ? 2 : 4;
    const uint32_t gstride = static_cast<uint32_t>(a.hv) * D * GS, qstride = static_cast<uint32_t>(a.hk) * D * ES;
    const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(
        reinterpret_cast<const unsigned char *>(a.g) + ((t0 * a.hv + h) * D) * GS, static_cast<uint32_t>(len) * gstride);
    const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(
        reinterpret_cast<const unsigned char *>(a.q) + ((t0 * a.hk + hk) * D) * ES, static_cast<uint32_t>(len) * qstride);
    const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(
        reinterpret_cast<const unsigned char *>(a.k) + ((t0 * a.hk + hk) * D) * ES, static_cast<uint32_t>(len) * qstride);
    int ch0 = 2 * cp;   // opaque: the per-row offsets are formed here, not hoisted by the caller's loop
    asm volatile("" : "+v"(ch0));
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
        const uint32_t row = static_cast<uint32_t>(grp * TPG + i);
        pg[i] = rd_pair<GATE_BF16>(rg, row * gstride + ch0 * GS);
        pq[i] = rd_pair<IN_BF16>(rq, row * qstride + ch0 * ES);
        pk[i] = rd_pair<IN_BF16>(rk, row * qstride + ch0 * ES);
    }
}

// v at rows 16 mt + 4 lq + r, column 16 nt + l16, one element per register
// as loaded (bf16, or f32 rounded at use), nothing computed on them here so
// that the loads stay in flight (zero past len).
template <int D, bool IN_BF16>
__device__ __forceinline__ void kda_fetch_v(const FwdArgs &a, int64_t t0, int len, int h, int nt, int lane,
                                            VRaw<IN_BF16> (&pv)[16]) {
    constexpr uint32_t ES = IN_BF16 ? 2 : 4;
    const int l16 = lane & 15, lq = lane >> 4;
    const uint32_t stride = static_cast<uint32_t>(a.hv) * D * ES;
    const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(
        reinterpret_cast<const unsigned char *>(a.v) + ((t0 * a.hv + h) * D) * ES, static_cast<uint32_t>(len) * stride);
    uint32_t voff = 4 * lq * stride + (16 * nt + l16) * ES;
    asm volatile("" : "+v"(voff));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t off = voff + static_cast<uint32_t>(16 * (j >> 2) + (j & 3)) * stride;
        if constexpr (IN_BF16) pv[j] = __builtin_bit_cast(__bf16, __builtin_amdgcn_raw_buffer_load_b16(rv, off, 0, 0));
        else pv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0));
    }
}
// beta of token t0 + lane (zero past len), as loaded
template <bool GATE_BF16>
__device__ __forceinline__ VRaw<GATE_BF16> fetch_beta(const FwdArgs &a, int64_t t0, int len, int h, int lane) {
    constexpr uint32_t GS = GATE_BF16 ? 2 : 4;
    const uint32_t stride = static_cast<uint32_t>(a.hv) * GS;
    const __amdgpu_buffer_rsrc_t rb = chunk_rsrc(
        reinterpret_cast<const unsigned char *>(a.beta) + (t0 * a.hv + h) * GS, static_cast<uint32_t>(len) * stride);
    if constexpr (GATE_BF16) return __builtin_bit_cast(__bf16, __builtin_amdgcn_raw_buffer_load_b16(rb, lane * stride, 0, 0));
    else return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * stride, 0, 0));
}

template <int D>
struct KdaLds {
    // Row pitches (bf16 elements).  The operand arrays and P are read as
    // 16-byte row fragments over key-permuted columns (kpos); k o e^{G_L - G}
    // with the transposing loads (4 rows of 32 bytes per 16 lanes) for the
    // state update; A and the diagonal inverses as 8-byte fragments, at
    // pitches of 2 mod 32 four-byte banks (16 lanes, one row each, no
    // conflict).  Measured: the 8-byte reads of q~ and k~ at a pitch of 8 mod
    // 32 banks cost twice the time of the whole A/P phase.
    static constexpr int PK = D + 16;              // operand arrays (key-permuted columns)
    static constexpr int PH = D + 16;              // k o e^{G_L - G}
    static constexpr int PP = C + 4;               // A
    static constexpr int PQ = C + 16;              // P (key-permuted columns)
    static constexpr int PD = 20;
    static constexpr int oQt = 0;                  // q~ [64][PK] (block references)
    static constexpr int oKt = oQt + C * PK * 2;   // k~
    static constexpr int oQs = oKt + C * PK * 2;   // q o e^G [64][PK] (the chunk start as reference)
    static constexpr int oKs = oQs + C * PK * 2;   // k o e^G
    static constexpr int oKh = oKs + C * PK * 2;   // k o e^{G_L - G} [64][PH] (the state update's)
    // column copies k^(b), b = 0..3: rows 0 .. 16 b + 15 of copy b at row 8 b (b + 1)
    static constexpr int oKc = oKh + C * PH * 2;
    static constexpr int oA = oKc + 160 * PK * 2;  // diag(b) A~ strictly lower [i][j]; the scan's group totals before
    static constexpr int oP = oA + C * PP * 2;     // scale tril(q~ k^^T) [i][kpos(j)]
    static constexpr int oDi = oP + C * PQ * 2;    // inverses of the diagonal blocks [4][16][PD]
    static constexpr int oV = oDi + 4 * 16 * PD * 2;   // f32 [D] e^{G_L}; [64] b
    static constexpr int NG = 2 * kKdaThreads / D; // token groups of the gate scan (a thread: 2 channels)
    static constexpr int oTot = oA;                // f32 [NG][D] group totals of the scan (A's space, free then)
    static constexpr int bytes = oV + (D + C) * 4;
    static_assert(NG * D * 4 <= C * PP * 2, "the group totals fit in A's space");
    static_assert(16 % (C / NG) == 0, "a scan group's tokens lie in one 16-row block");
};

template <int D, bool IN_BF16, bool GATE_BF16>
__global__ void __launch_bounds__(kKdaThreads) gdr_kda_fwd_kernel(FwdArgs a) {
    using Ly = KdaLds<D>;
    constexpr int PK = Ly::PK, PH = Ly::PH, PP = Ly::PP, PQ = Ly::PQ, PD = Ly::PD, NG = Ly::NG;
    constexpr int TPG = C / NG;     // tokens per scan group
    constexpr int MT = D / 16;      // dk tiles
    constexpr int NTD = D / 16;     // dv tiles (one per wave while wave < NTD)
    extern __shared__ __align__(16) unsigned char lds[];
    uint16_t *sQt = reinterpret_cast<uint16_t *>(lds + Ly::oQt);
    uint16_t *sKt = reinterpret_cast<uint16_t *>(lds + Ly::oKt);
    uint16_t *sQs = reinterpret_cast<uint16_t *>(lds + Ly::oQs);
    uint16_t *sKs = reinterpret_cast<uint16_t *>(lds + Ly::oKs);
    uint16_t *sKh = reinterpret_cast<uint16_t *>(lds + Ly::oKh);
    uint16_t *sKc = reinterpret_cast<uint16_t *>(lds + Ly::oKc);
    uint16_t *sA = reinterpret_cast<uint16_t *>(lds + Ly::oA);
    uint16_t *sP = reinterpret_cast<uint16_t *>(lds + Ly::oP);
    uint16_t *sDi = reinterpret_cast<uint16_t *>(lds + Ly::oDi);
    float *sEL = reinterpret_cast<float *>(lds + Ly::oV);
    float *sB = sEL + D;
    float *sTot = reinterpret_cast<float *>(lds + Ly::oTot);
    auto kcopy = [&](int b) { return sKc + 8 * b * (b + 1) * PK; };   // column copy k^(b)

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
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform branches
    const bool colwave = wave < NTD;
    const int nt = wave;
    const int64_t nch = (eos - bos + C - 1) / C;

    // the state: rows dk (tile mt, row 4 lq + r), columns 16 nt + l16
    f32x4 H[MT];
    {
        const int lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                H[mt][r] = (colwave && a.h0) ? a.h0[((n * a.hv + h) * D + 16 * mt + 4 * lq + r) * D + 16 * nt + l16] : 0.f;
    }

    // Registers of the next chunk, loaded while the current one is processed:
    // this thread's channel of g, q and k over its TPG tokens, its wave's v
    // values (rows 4 lq + r of the four token blocks, column 16 nt + l16) and
    // beta of its lane's token, each as loaded.
    const int cp = tid % (D / 2), grp = tid / (D / 2), ch = 2 * cp, chp = kpos(ch);   // channels ch, ch + 1
    PRaw<GATE_BF16> pg[TPG];
    PRaw<IN_BF16> pq[TPG], pk[TPG];
    VRaw<IN_BF16> pv[16];
    VRaw<GATE_BF16> pb = 0;
    // Unconditional: past the last chunk the ranges are empty and read zeros
    // (a branch here would make the compiler wait for the loads at its join).
    // Two parts issued in different phases, so that no more loads are in
    // flight per wave than its counter of outstanding loads (63) can track.
#define GDR_KDA_RANGE(cc)                                                                               \
    const int64_t t0_ = bos + C * (cc);                                                                 \
    const int64_t r_ = eos - t0_;                                                                       \
    const int len_ = static_cast<int>(r_ <= 0 ? 0 : r_ < C ? r_ : C);                                   \
    const int ln_ = tid & 63;
#define GDR_KDA_FETCH_G(cc)                                                                             \
    {                                                                                                   \
        GDR_KDA_RANGE(cc)                                                                               \
        kda_fetch_gate<D, TPG, IN_BF16, GATE_BF16>(a, t0_, len_, h, hk, cp, grp, pg, pq, pk);          \
        (void)ln_;                                                                                      \
    }
#define GDR_KDA_FETCH_V(cc)                                                                             \
    {                                                                                                   \
        GDR_KDA_RANGE(cc)                                                                               \
        if (D == 128 || colwave) kda_fetch_v<D, IN_BF16>(a, t0_, len_, h, nt, ln_, pv);                 \
        pb = fetch_beta<GATE_BF16>(a, t0_, len_, h, ln_);                                               \
    }
    GDR_KDA_FETCH_G(0)
    GDR_KDA_FETCH_V(0)
    // P's blocks above the diagonal are read (by P U) but never written: zero
    // them once (all of P).  A's are neither read nor written.
    for (int i = tid; i < C * PQ / 8; i += kKdaThreads) reinterpret_cast<v4u32 *>(sP)[i] = v4u32{0u, 0u, 0u, 0u};

    for (int64_t c = 0; c < nch; ++c) {
        int lane = tid & 63;   // opaque per iteration: keeps per-lane addresses inside the loop
        asm volatile("" : "+v"(lane));
        const int l16 = lane & 15, lq = lane >> 4;
        const int64_t t0 = bos + C * c;
        const int len = static_cast<int>(eos - t0 < C ? eos - t0 : C);

        // ---- gates: per-channel prefix sums (log2 units), two channels over TPG
        // tokens per thread
        float G2[2][TPG];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                run += pair_val<GATE_BF16>(pg[i], e) * kLog2e;
                G2[e][i] = run;
            }
        }
        __syncthreads();   // the previous chunk's reads of LDS are done (A's space takes the totals)
        *reinterpret_cast<float2 *>(sTot + grp * D + ch) = float2{G2[0][TPG - 1], G2[1][TPG - 1]};
        if (wave == 0) sB[lane] = static_cast<float>(pb);
        __syncthreads();
        {
            // offsets of this thread's tokens, the block references R_b (G at
            // the row before block b, R_0 = 0) and G_L, per channel (log2 units)
            constexpr int NB = C / 16;
            float offs[2] = {0.f, 0.f}, gl[2] = {0.f, 0.f}, rb[2][NB] = {};
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const float2 tj = *reinterpret_cast<const float2 *>(sTot + j * D + ch);
                offs[0] += j < grp ? tj.x : 0.f;
                offs[1] += j < grp ? tj.y : 0.f;
#pragma unroll
                for (int b = 1; b < NB; ++b) {
                    rb[0][b] += j < 16 * b / TPG ? tj.x : 0.f;
                    rb[1][b] += j < 16 * b / TPG ? tj.y : 0.f;
                }
                gl[0] += tj.x;
                gl[1] += tj.y;
            }
            if (grp == 0) {
#pragma unroll
                for (int e = 0; e < 2; ++e) sEL[ch + e] = fast_exp2(gl[e]);
            }
            // the 16-row block of this thread's tokens (one per wave)
            const int blk = __builtin_amdgcn_readfirstlane(grp * TPG / 16);
            // per channel: R_blk, e^{R_blk} and e^{R_b - R_blk} for the later blocks (all <= 1)
            float rbb[2], eb[2], ratio[2][NB];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                rbb[e] = rb[e][0];
#pragma unroll
                for (int b = 1; b < NB; ++b) rbb[e] = b == blk ? rb[e][b] : rbb[e];
                eb[e] = fast_exp2(rbb[e]);
#pragma unroll
                for (int b = 0; b < NB; ++b) ratio[e][b] = fast_exp2(fminf(rb[e][b] - rbb[e], 0.f));
            }
            bool out_of_range = false;
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                const int row = grp * TPG + i;
                float x[2], qv[2], kv[2], er[2], ed[2], eu[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    x[e] = G2[e][i] + offs[e];   // G at this row
                    qv[e] = static_cast<float>(static_cast<__bf16>(pair_val<IN_BF16>(pq[i], e)));
                    kv[e] = static_cast<float>(static_cast<__bf16>(pair_val<IN_BF16>(pk[i], e)));
                    // e^{G - R_blk} (<= 1), e^{R_blk - G} (>= 1, the diagonal block's), e^{G_L - G} (<= 1)
                    er[e] = fast_exp2(x[e] - rbb[e]);
                    ed[e] = fast_exp2(rbb[e] - x[e]);
                    eu[e] = fast_exp2(gl[e] - x[e]);
                    // the largest factor, e^{R_blk - G} inside the block, must stay finite
                    out_of_range |= rbb[e] - x[e] > 126.f;
                }
                // the two channels' bf16 values, packed; channels ch, ch + 1 stay
                // adjacent under kpos (ch is even).  q~, k~ (block reference),
                // q, k o e^G (chunk start), k o e^{G_L - G}, the column copies k^(b)
                auto pk2 = [](float lo, float hi) { return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo, (__bf16)hi}); };
                *reinterpret_cast<uint32_t *>(sQt + row * PK + chp) = pk2(qv[0] * er[0], qv[1] * er[1]);
                *reinterpret_cast<uint32_t *>(sKt + row * PK + chp) = pk2(kv[0] * er[0], kv[1] * er[1]);
                *reinterpret_cast<uint32_t *>(sQs + row * PK + chp) = pk2(qv[0] * er[0] * eb[0], qv[1] * er[1] * eb[1]);
                *reinterpret_cast<uint32_t *>(sKs + row * PK + chp) = pk2(kv[0] * er[0] * eb[0], kv[1] * er[1] * eb[1]);
                *reinterpret_cast<uint32_t *>(sKh + row * PH + ch) = pk2(kv[0] * eu[0], kv[1] * eu[1]);
                const float kd0 = kv[0] * ed[0], kd1 = kv[1] * ed[1];
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b >= blk)   // wave-uniform
                        *reinterpret_cast<uint32_t *>(kcopy(b) + row * PK + chp) = pk2(kd0 * ratio[0][b], kd1 * ratio[1][b]);
            }
            if (out_of_range)
                __hip_atomic_fetch_or(a.status, kDevStatKdaRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        VRaw<IN_BF16> cv[16];   // this chunk's v values; the registers above take the next chunk
#pragma unroll
        for (int j = 0; j < 16; ++j) cv[j] = pv[j];
        GDR_KDA_FETCH_G(c + 1)
        __syncthreads();

        // ---- blocks of A = diag(b) k~ k^^T (strictly lower) and of P = scale q~ k^^T
        // (lower): waves 0-3 take diagonal block b = wave of A, its inverse, then
        // block wave of P; waves 4-7 share the six blocks of A below the diagonal
        // and the other six blocks of P (three each)
        {
            const bool dw = wave < 4;
            // tile t: A blocks 0..5 below the diagonal, then P blocks (t - 2) for t = 6..11
            auto tile = [&](bool ka, int bi, int bj) __attribute__((always_inline)) {
                const uint16_t *Am = ka ? sKt : sQt;
                const uint16_t *Bm = kcopy(bi);   // the column copy of row block bi's reference
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < D; k0 += 32)
                    acc = mfma32(kfrag8(Am, PK, 16 * bi, k0, l16, lq), kfrag8(Bm, PK, 16 * bj, k0, l16, lq), acc);
                const int j = 16 * bj + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * bi + 4 * lq + r;
                    if (ka) sA[i * PP + j] = bf16_bits(j < i ? sB[i] * acc[r] : 0.f);
                    else sP[i * PQ + kpos(j)] = bf16_bits(j <= i ? a.scale * acc[r] : 0.f);
                }
            };
            auto ptile = [&](int tt) __attribute__((always_inline)) {
                const int bi = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;
                tile(false, bi, tt - bi * (bi + 1) / 2);
            };
            if (dw) {
                tile(true, wave, wave);
                // inverse of diagonal block b of I + A, column l16 by fp32 forward
                // substitution over the bf16 values this wave has just stored
                lds_wait();
                const int b = wave;
                float x[16];
                x[0] = l16 == 0 ? 1.f : 0.f;
#pragma unroll
                for (int i = 1; i < 16; ++i) {
                    float s = i == l16 ? 1.f : 0.f;
#pragma unroll
                    for (int m4 = 0; m4 < i; m4 += 4) {
                        // entries m4 .. m4 + 3 of row i, one 8-byte read (the same for all lanes)
                        const v2u32 w = *reinterpret_cast<const v2u32 *>(sA + (16 * b + i) * PP + 16 * b + m4);
                        const float am[4] = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                             __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (m4 + u < i) s -= am[u] * x[m4 + u];
                    }
                    x[i] = s;
                }
                if (lq == 0) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) sDi[(16 * b + i) * PD + l16] = bf16_bits(x[i]);
                }
                ptile(wave);
            } else {
                for (int t = wave - 4; t < 12; t += 4) {
                    if (t < 6) {
                        const int bi = t >= 3 ? 3 : t >= 1 ? 2 : 1;
                        tile(true, bi, t - (bi - 1) * bi / 2);
                    } else {
                        ptile(t - 2);
                    }
                }
            }
        }
        // ---- then (k o e^G) H and ((q o e^G) H)^T for this wave's dv tile,
        // H taken from the wave's own state registers
        f32x4 X[4], QS[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[mt] = QS[mt] = zero4();
        if (colwave) {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const bf16x8 bs = cat(cvt4(H[2 * kk]), cvt4(H[2 * kk + 1]));
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    X[mt] = mfma32(kfrag8(sKs, PK, 16 * mt, 32 * kk, l16, lq), bs, X[mt]);
                    QS[mt] = mfma32(bs, kfrag8(sQs, PK, 16 * mt, 32 * kk, l16, lq), QS[mt]);   // ((q o e^G) H)^T
                }
            }
        }
        GDR_KDA_FETCH_V(c + 1)
        __syncthreads();

        // ---- U = (I + A)^-1 diag(b) (V - X) by block forward substitution,
        // U_b = D_b (W_b - sum_{c<b} A_bc U_c); O^T = scale (q~ S_m)^T + (P U)^T, with
        // the register tiles of S_m and U as A operands (so a lane holds four dv of
        // one token: one 8-byte store); H update (dv tile nt)
        if (colwave) {
            bf16x4 ub[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f32x4 e;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * b + 4 * lq + r;
                    const float vv = static_cast<float>(static_cast<__bf16>(cv[4 * b + r]));
                    e[r] = sB[i] * (vv - X[b][r]);
                }
#pragma unroll
                for (int cc = 0; cc < 3; ++cc)
                    if (cc < b) e = mfma16z(ld4(sA + (16 * b + l16) * PP + 16 * cc + 4 * lq), neg4(ub[cc]), e);
                ub[b] = cvt4(mfma16z(ld4(sDi + (16 * b + l16) * PD + 4 * lq), cvt4(e), zero4()));
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) QS[mt] = QS[mt] * a.scale;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 bu = cat(ub[2 * kk], ub[2 * kk + 1]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) QS[mt] = mfma32(bu, kfrag8(sP, PQ, 16 * mt, 32 * kk, l16, lq), QS[mt]);   // (P U)^T
            }
            // O^T tiles: lane (l16, lq) holds token 16 mt + l16, dv 16 nt + 4 lq .. + 3
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int i = 16 * mt + l16;
                if (i < len) {
                    const int64_t oi = ((t0 + i) * a.hv + h) * D + 16 * nt + 4 * lq;
                    if constexpr (IN_BF16) *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint16_t *>(a.o) + oi) = cvt4(QS[mt]);
                    else *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.o) + oi) = QS[mt];
                }
            }
            // H <- diag(e^{G_L}) H + (k o e^{G_L - G})^T U
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 R = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    R = mfma32(kfrag_cols(sKh, PH, 16 * mt, 32 * kk, l16, lq), cat(ub[2 * kk], ub[2 * kk + 1]), R);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mt + 4 * lq + r;
                    H[mt][r] = sEL[row] * H[mt][r] + R[r];
                }
            }
        }
    }

    if (a.ht && colwave) {
        const int lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
        float *dst = a.ht + (n * a.hv + h) * D * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * mt + 4 * lq + r) * D + 16 * nt + l16] = H[mt][r];
    }
#undef GDR_KDA_FETCH_G
#undef GDR_KDA_FETCH_V
#undef GDR_KDA_RANGE
}

template <int D, bool IN_BF16, bool GATE_BF16>
hipError_t launch_kda_t(const FwdArgs &a, hipStream_t stream) {
    auto kern = gdr_kda_fwd_kernel<D, IN_BF16, GATE_BF16>;
    const int lds = KdaLds<D>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.n_seq * a.hv)), dim3(kKdaThreads), lds, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_kda_d(const FwdArgs &a, hipStream_t s) {
    // f32 inputs run the fp32 token-serial kernel (launch_kda_fwd)
    if (!a.in_bf16) return hipErrorInvalidValue;
    return a.gate_bf16 ? launch_kda_t<D, true, true>(a, s) : launch_kda_t<D, true, false>(a, s);
}

static_assert(KdaLds<128>::bytes <= 160 * 1024, "KDA kernel LDS");

template <int D>
const void *kda_kernel(int gate_bf16) {
    return gate_bf16 ? reinterpret_cast<const void *>(gdr_kda_fwd_kernel<D, true, true>)
                     : reinterpret_cast<const void *>(gdr_kda_fwd_kernel<D, true, false>);
}

}  // namespace

hipError_t kda_slots(int d, int in_bf16, int gate_bf16, int *slots) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (!in_bf16) return hipErrorInvalidValue;   // f32 inputs run the fp32 kernel
    const void *kern = d == 64 ? kda_kernel<64>(gate_bf16) : kda_kernel<128>(gate_bf16);
    const int lds = d == 64 ? KdaLds<64>::bytes : KdaLds<128>::bytes;
    if ((e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kKdaThreads, lds)) != hipSuccess) return e;
    *slots = cus * per_cu;
    return hipSuccess;
}

hipError_t launch_kda_fwd(const FwdArgs &a, hipStream_t stream) {
    if (a.n_seq == 0 || a.hv == 0) return hipSuccess;
    if (!a.in_bf16) return launch_fwd_f32(a, true, stream);   // f32 inputs: fp32 arithmetic
    return a.d == 64 ? launch_kda_d<64>(a, stream) : launch_kda_d<128>(a, stream);
}

}  // namespace gdr
