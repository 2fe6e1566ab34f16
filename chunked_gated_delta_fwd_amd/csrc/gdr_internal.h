// Internal interface between the host API (gdr_api.cpp) and the kernels
// (gdr_kernels.hip).  Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// Everything a fused-forward launch needs, already validated on the host.
struct FwdArgs {
    const void *q, *k, *v, *g, *beta;
    const int32_t *cu;      // NULL: fixed-length rows
    const int32_t *order;   // NULL: natural order
    const float *h0;        // NULL: zero state
    void *o;                // NULL: not written
    float *ht;              // NULL: not written
    int64_t n_seq;          // N
    int64_t seq_len;        // T per row when cu == NULL
    int64_t total_tokens;   // rows of q/k/v/o (B * T); bounds every token index
    int32_t hk, hv, d;      // d: key head dim dk
    int32_t dv;             // value head dim (64 or 128)
    int32_t in_bf16;        // q/k/v/o dtype: 1 bf16, 0 f32
    int32_t gate_bf16;      // g/beta dtype
    float scale;
    // chunk-boundary states (NULL: not written): row ck_offs[n] + c (or
    // n * ceil(seq_len / 64) + c for fixed-length rows) of [ck_rows, Hv, d, d],
    // fp32 [dk][dv] into hck or, when hck16 is set instead, bf16 (rounded to
    // nearest even) into hck16 in the forward kernel's tile order: 8-byte
    // piece ((w * d/16 + kb) * (d/64) + nt) * 64 + lane holds rows
    // 32 (kb/2) + 8 (lane/16) + 4 (kb%2) + 0..3 of column
    // w d/4 + (d/16) (lane%16 / 4) + 4 nt + lane%4 (w = chain wave 0..3)
    float *hck;
    uint16_t *hck16;
    const int32_t *ck_offs;
    int64_t ck_rows;
    // fp32 checkpoints (hck) every ck_every tokens (a multiple of 16; 64 gives
    // the chunk-boundary states above): row ck_offs[n] + j (ck_offs then holds
    // prefix sums of ceil(L / ck_every); fixed-length rows: n * ceil(seq_len /
    // ck_every) + j) receives the state after min((j+1) ck_every, L) tokens
    int32_t ck_every;
    // device status word (sticky error bits, see kDevStat*) and the number of
    // polls after which a hand-off wait between the kernel's two wave roles
    // gives up (it then sets kDevStatWaitTimeout and poisons ht with NaN)
    uint32_t *status;
    int32_t spin_max;
};

// Bits of the per-device status word the kernels set (sticky until cleared).
constexpr uint32_t kDevStatWaitTimeout = 1u;   // a hand-off wait gave up: outputs of that call are wrong
constexpr uint32_t kDevStatKdaRange = 2u;      // per-channel gates beyond the range of their chunk form
constexpr int32_t kSpinDefault = 1 << 18;      // polls (each s_sleep 1, about 64 cycles) before giving up

// Per-device memory the library keeps in static device arrays: the status
// word and the scratch of the no-allocation entry point.  Addresses come from
// hipGetSymbolAddress for the current device, once per device.
constexpr size_t kScratchBytes = 64 * 1024;
hipError_t device_buffers(uint32_t **status, void **scratch);

// Device-side check of the cu_seqlens preconditions (cu[0] == 0, non-decreasing,
// cu[N] == total): writes result[0..3] = {kind, index, value, value}, kind 0
// when the content is valid (1: cu[0] != 0, 2: cu[i+1] < cu[i], 3: cu[N] != total).
hipError_t launch_check_cu(const int32_t *cu, int64_t n_seq, int64_t total, int32_t *result,
                           hipStream_t stream);

// One recurrent step per (sequence, v-head), already validated on the host.
struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    float *h;               // [B, Hv, d, d] fp32, updated in place
    void *o;                // [B, Hv, d]
    int64_t batch;          // B
    int32_t hk, hv, d;      // d: key head dim dk
    int32_t dv;             // value head dim
    int32_t in_bf16, gate_bf16;
    float scale;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// Dynamic LDS bytes (they depend on dk only) and threads per work-group of
// the fused forward kernel (4 state-chain waves + 4 preparation waves).
int fwd_lds_bytes(int dk);
constexpr int kFwdThreads = 512;
// Threads and static LDS bytes of the token-serial fp32 kernel (f32 inputs).
constexpr int kFwdF32Threads = 256;
int fwd_f32_lds_bytes(int dk, int dv);
constexpr int kChunk = 64;

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);
// Per-channel gates: the same arguments with g of shape [tokens, Hv, d].
hipError_t launch_kda_fwd(const FwdArgs &a, hipStream_t stream);
// f32 q/k/v/o: the token-serial fp32 kernel (launch_fwd and launch_kda_fwd
// route f32 inputs here; hck16 must be NULL).  per_channel: g is [tokens, Hv, d].
hipError_t launch_fwd_f32(const FwdArgs &a, bool per_channel, hipStream_t stream);

// chunk_offsets: prefix sums of ceil(L / unit) (unit = kChunk for chunk
// indices; the chunk map requires unit = kChunk).
hipError_t launch_prepare(const int32_t *cu, int64_t n_seq, int32_t *chunk_offsets,
                          int32_t *chunk_map, int64_t nt_max, int32_t *order,
                          hipStream_t stream, int32_t unit = kChunk);

// Dispatch order for few sequences (1 <= n_seq <= 64) on `groups` (<= 16)
// machines of CUs; see the kernel for the model.
hipError_t launch_order(const int32_t *cu, int64_t n_seq, int32_t groups, int32_t *order,
                        hipStream_t stream);
// Work-groups of the fused forward kernel resident on the device at once.
hipError_t fwd_slots(int dk, int dv, int in_bf16, int gate_bf16, int *slots);
// Work-groups of the per-channel-gate forward kernel resident at once.
hipError_t kda_slots(int d, int in_bf16, int gate_bf16, int *slots);

// chunk_map != NULL: varlen (grid nt_max); else n_rows fixed rows of seq_len tokens.
hipError_t launch_cumsum(const void *g, int gate_bf16, const int32_t *cu,
                         const int32_t *chunk_map, int64_t nt_max, int64_t n_rows,
                         int64_t seq_len, int64_t total_tokens, int32_t heads, float *G,
                         hipStream_t stream);

// Everything the backward kernels need, already validated on the host.  The
// forward recompute (states after every chunk, into hck) is launched first by
// the caller with the forward kernel.
struct BwdArgs {
    const void *q, *k, *v, *g, *beta, *dout;
    const int32_t *cu;      // NULL: fixed-length rows
    const int32_t *map;     // chunk row -> (sequence, chunk) pairs; NULL for fixed-length rows
    const int32_t *offs;    // first chunk row of each sequence; NULL for fixed-length rows
    const int32_t *order;   // start order of the reverse chain; NULL: natural
    const float *h0;        // NULL: zero initial state
    const float *dht;       // NULL: zero gradient of the final state
    const uint16_t *hck;    // forward state after every chunk [rows, Hv, d*d], bf16 in the forward's tile order (FwdArgs::hck16)
    uint16_t *tmat;         // per chunk: T^T, T = (I + diag(b) A~)^-1, bf16 [rows, Hv, 64, 64]
    uint16_t *du;           // per chunk: dU, bf16 [rows, Hv, 64 * d] in 16x16 tiles, lane-major
    // per chunk: gradient of the state at its end, bf16 [rows, Hv, d*d] in the
    // chain kernel's tile order: 8-byte piece ((w * d/16 + mt) * (d/64) + nt) * 64
    // + lane holds rows 16 mt + 4 (lane/16) + 0..3 of column w d/4 + 16 nt + lane%16
    uint16_t *dhe;
    void *dq, *dk, *dv;     // dtype of q
    float *dg, *dbeta;
    float *dh0;             // NULL: not written
    int64_t n_seq, seq_len, total_tokens, rows;
    int32_t hk, hv, d, in_bf16, gate_bf16;
    float scale;
};
// Per-chunk preparation, reverse chain over chunks, per-chunk gradients.
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);

hipError_t launch_selftest_mfma(const uint16_t *a, const uint16_t *b, float *c,
                                hipStream_t stream);

}  // namespace gdr
