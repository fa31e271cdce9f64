// kernels.h -- internal launch interface between the host layer (mllm.cpp)
// and the gfx950 kernels (decode.hip, prefill.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mllm {

constexpr int kMaxHalfDim = 64;  // D / 2 for the largest supported head size (128)
constexpr int kMaxPrefillOrder = 256;  // entries a prefill schedule can reorder

// Everything one decode step needs, resolved and validated by the host layer.
struct DecodeParams {
    const uint16_t *q;      // [A, Hq, D] 16-bit codes, strides q_sa / q_sh (elements)
    const uint16_t *k_new;  // [A, Hkv, D]
    const uint16_t *v_new;  // [A, Hkv, D]
    int64_t q_sa, q_sh, kn_sa, kn_sh, vn_sa, vn_sh;
    const int32_t *positions;  // [A] device
    const int32_t *rows;       // [A] device
    uint16_t *kc;              // layer K block [S, C, Hkv, D], dense
    uint16_t *vc;              // layer V block
    uint16_t *out;             // [A, Hq, D]
    int64_t o_sa, o_sh;
    float *qrot;      // workspace [A, Hq, D]      rotated queries, FP32
    float *part_o;    // workspace [slots, G, D]  per (segment, group, head) unnormalized outputs
    float *part_ml;   // workspace [slots, G, 2]  per (segment, group, head) (max, sum), log2 domain
    long long *plan;  // workspace [A + 2]: plan units before each entry, then the tile and segment totals
    int32_t *status;  // optional device status word
    int32_t dtype;     // storage type of every 16-bit tensor: 1 BF16, 2 FP16
    int32_t A, S, C, Hq, Hkv, D, G;
    int32_t NS;        // work groups of the decode launch
    int32_t plan_weighted;  // 1: the launch holds two resident groups per compute unit
                            // (the first-dispatched half gets more work, see make_plan)
    int32_t plan_wa, plan_wb;  // work weights of the first and second half when weighted
    int32_t HG, NHG;   // kv heads per group (one wave each), head groups per entry
    float scale_log2;  // log2(e) / sqrt(D)
    float inv_freq[kMaxHalfDim];
};

// Workspace carve-up for a decode step (all offsets 256-byte aligned).
struct DecodeWorkspace {
    uint64_t qrot_off, part_o_off, part_ml_off, plan_off, total;
};
DecodeWorkspace decode_workspace_layout(int64_t A, int64_t Hq, int64_t Hkv, int64_t D,
                                        int64_t NS);

// RoPE(K) + K/V store + RoPE(Q) -> qrot.  One block per active entry.
hipError_t launch_rope_store(const DecodeParams &p, hipStream_t stream);
// Tuned decode step: RoPE + store + split-K attention + merge in one launch.
// e0 / e1: optional events stamped at the kernel's start and end.
hipError_t launch_decode_fused(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                               hipEvent_t e1);
// kv heads per work group for a head layout (a power of two dividing Hkv).
int decode_head_group(int Hkv, int G);
// Resident work groups of the decode kernel variant on a device (0 on error).
int decode_resident_groups(int device, int D, int G, int HG, int dtype);
// Cross-wave merge -> output in the storage type (one wave per entry and query head).
hipError_t launch_decode_merge(const DecodeParams &p, hipStream_t stream);
// Readable one-wave-per-(entry, query head) attention straight to the output.
hipError_t launch_decode_readable(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                                  hipEvent_t e1);

struct PrefillParams {
    const uint16_t *q;      // [A, T, Hq, D]
    const uint16_t *k_new;  // [A, T, Hkv, D]
    const uint16_t *v_new;  // [A, T, Hkv, D]
    int64_t q_sa, q_st, q_sh, kn_sa, kn_st, kn_sh, vn_sa, vn_st, vn_sh;
    const int32_t *rows;    // [A] device
    const int32_t *starts;  // [A] device first position of each entry's chunk (NULL: all 0)
    const int32_t *lens;    // [A] device tokens of each entry, 1 .. T (NULL: all T)
    uint16_t *kc, *vc;      // layer blocks [S, C, Hkv, D]
    uint16_t *out;          // [A, T, Hq, D]
    int64_t o_sa, o_st, o_sh;
    float2 *table;          // workspace [A, T, D/2] (cos, sin) of position starts[a] + t
    int32_t dtype;          // storage type of every 16-bit tensor: 1 BF16, 2 FP16
    int32_t A, T, S, C, Hq, Hkv, D, G;
    float scale_log2;
    float inv_freq[kMaxHalfDim];
    // the order in which the matrix-core kernel takes the entries (a schedule
    // only): heaviest first for a chunk of mixed starts and lengths, so no long
    // cached prefix starts last; n_order = 0 takes them in index order
    int32_t n_order;
    uint16_t order[kMaxPrefillOrder];
};
// fills p.n_order / p.order from the host copies of the chunk's starts and
// lengths (starts == NULL: the equal-length prefill, index order)
void prefill_order(PrefillParams &p, const int32_t *starts_host, const int32_t *lens_host);
uint64_t prefill_workspace_bytes(int64_t A, int64_t T, int64_t Hq, int64_t D);
// RoPE(K) + K/V store, then attention: kernel 0 = matrix-core tiles, 1 = readable.
// e0 / e1: optional events stamped at the attention kernel's start and end.
hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream, int kernel, hipEvent_t e0,
                          hipEvent_t e1);

}  // namespace mllm
