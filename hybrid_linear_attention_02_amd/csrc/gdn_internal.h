// Internal declarations shared by the translation units of libgdn.so.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>
#include <set>

#include "gdn.h"

struct gdn_pool {
    int32_t num_slots = 0;
    int32_t num_v_heads = 0;
    int32_t dk = 0;
    int32_t dv = 0;
    float* storage = nullptr;          // caller-owned device memory
    std::vector<int32_t> ref;          // refcount per slot (0 = free)
    std::set<int32_t> free_slots;      // ordered: lowest index first
};

namespace gdn {

// Record a failure message for gdn_last_error() and return `code`.
int fail(int code, const std::string& msg);

// Kernel launchers (defined in the .hip files). They assume validated
// arguments and return GDN_OK or GDN_E_HIP / GDN_E_UNSUPPORTED.
// `storage` (when not NULL) replaces the pool's own slot storage: a tensor of
// the same [slot][HV][dk][dv] shape, as one layer of a stack of GDN layers
// that share the pool's slot numbering holds.
int launch_decode(const gdn_pool* pool, const gdn_decode_args* a, void* stream, float* storage = nullptr);
int check_decode_args(const gdn_pool* pool, const gdn_decode_args* a, const char* fn);
constexpr int kMaxDraft = 64;     // draft tokens per request in one verify launch
int launch_verify(const gdn_pool* pool, const gdn_verify_args* a, void* stream);
int launch_transfer(const gdn_pool* pool, bool pack, int32_t n, const int32_t* slots, float* buffer,
                    int32_t* err_flag, void* stream);

// Sequence split of long prefills. A sequence of more than seg_len chunks is
// cut into segments of seg_len chunks; each segment's local end state E and
// transition M (the dk x dk map the segment applies to its initial state) are
// computed for all segments at once, chained across segments, and the
// segments then run their outputs in parallel from their true initial
// states. It costs about twice the work of one pass, so it is used only when
// one pass would leave most of the chip idle; choose_seg_len picks the length.
constexpr int kNumCUs = 256;      // MI355X compute units
int32_t choose_seg_len(const int32_t* cu_host, int32_t n, int32_t hv, int32_t dk, int32_t dv);

// Compute waves (16 value columns each) per workgroup of the bf16
// recurrence: the output pass takes min(dv, 64) columns per workgroup, the
// state pass at most dk of them, so that its dk transition columns split
// into whole groups too.
inline int prefill_output_waves(int dv) { return dv >= 64 ? 4 : dv / 16; }
// dk the bf16 prefill kernels run at: dk = 16 runs at 32 (the MFMA k-step),
// with q and k zero-padded and the pool tiles' 16 rows read and written only.
inline int prefill_kernel_dk(int dk) { return dk < 32 ? 32 : dk; }
inline int prefill_state_waves(int dk, int dv) {
    const int nw = prefill_output_waves(dv);
    return nw * 16 <= dk ? nw : dk / 16;
}

struct PrefillPlan {
    int32_t num_chunks = 0;       // sum over sequences of ceil(len / 64)
    int32_t seg_len = 0;          // chunks per segment, 0 = no split (one segment per sequence)
    int32_t num_segs = 0;         // total segments
    size_t off_chunk_offsets = 0; // int32 [N+1]: first chunk of each sequence
    size_t off_seg_offsets = 0;   // int32 [N+1]: first segment of each sequence
    size_t off_tp = 0;            // T and P: bf16 [chunks][HV][2][64 * 64] row-operand fragments, or for
                                  // float32 inputs fp32 [chunks][HV][2][10][64][4] block fragments
    size_t off_sc = 0;            // float [chunks][HV][5][64]: per-token scale rows
    size_t off_se = 0;            // float [segs][HV][dk][dv]: local end state E (split only)
    size_t off_sm = 0;            // bf16 [segs][HV][2][dk][dk]: transition M, high then low part (split only)
    size_t off_sh = 0;            // float [segs][HV][dk][dv]: segment initial states (split only)
    size_t bytes = 0;
};
int plan_prefill(const gdn_pool* pool, const gdn_prefill_args* a, PrefillPlan* plan);
// bf16 inputs: chunked form on the bf16 MFMA; float32 inputs: chunked form
// on the fp32 MFMA
int launch_prefill(const gdn_pool* pool, const gdn_prefill_args* a, const PrefillPlan& plan,
                   void* workspace, void* stream);

}  // namespace gdn
