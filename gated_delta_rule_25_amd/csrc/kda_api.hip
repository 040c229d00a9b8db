// kda_api.hip — the extern "C" boundary of libkda.so (declared in include/kda.h).
//
// Host side only: argument validation (before anything is enqueued), the
// launch plan, and the launches on the caller's stream.  No device memory is
// allocated and the host never waits on the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

constexpr int kD = 128;

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Range range_of(const void* p, size_t bytes) {
  Range r;
  if (p && bytes) {
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + bytes;
  }
  return r;
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

int cu_count_for_current_device() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

size_t elem_size(kda_dtype dt) { return dt == KDA_DTYPE_BF16 ? 2 : 4; }

bool dtype_ok(kda_dtype dt) { return dt == KDA_DTYPE_F32 || dt == KDA_DTYPE_BF16; }

// q, k, v, log_alpha, gate, o and the states move as 16-byte vectors; the
// rest (beta, cu_seqlens, conv and norm weights, workspace) are read as scalars.
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMinAutoSegment = 512;
#ifndef KDA_PREP_CHUNKS_PER_BLOCK
#define KDA_PREP_CHUNKS_PER_BLOCK 8
#endif
constexpr int kPrepChunksPerBlock = KDA_PREP_CHUNKS_PER_BLOCK;

// Segment length of the segmented schedule, or 0 for the sequential one.
// Automatic choice: only when the sequential schedule's workgroups fill less
// than a third of the compute units; then enough segments to fill them once
// (the segmented form does about twice the state work, so it pays from about
// three segments per chain on).
int64_t choose_segment_tokens(int num_seqs, int64_t total_tokens, int num_heads, const kda_fused_opts& f,
                              int cus) {
  if (f.segment_tokens < 0) return 0;
  if (f.segment_tokens > 0) return f.segment_tokens;
  const int64_t per_chain = f.gate ? 1 : 2;  // workgroups per (sequence, head)
  const int64_t blocks = (int64_t)num_seqs * num_heads * per_chain;
  if (3 * blocks > cus) return 0;
  const int64_t target = (cus + num_heads * per_chain - 1) / (num_heads * per_chain);
  int64_t seg = (total_tokens + target - 1) / target;
  seg = (seg + 63) / 64 * 64;
  if (seg < kMinAutoSegment) seg = kMinAutoSegment;
  if ((int64_t)num_seqs * seg >= total_tokens) return 0;  // sequences already about one segment long
  return seg;
}

// Factor store budget of the two-kernel schedule; longer inputs run in
// several windows.  kda_fused_opts::factor_budget_mib sets a smaller budget.
// 16 GiB, under 6 % of the GPU's HBM: every window reloads and rewrites the
// state of each (sequence, head) and pays the kernels' ramp and tail, so
// fewer windows are faster (measured against 4 GiB: long context 2 % and
// the fused varlen batch 3 % faster, with 1 and 8 windows instead of 4 and 29).
constexpr int64_t kFactorBudgetMiB = 16384;

size_t factor_budget(const kda_fused_opts& f) {
  const int64_t mib = f.factor_budget_mib > 0 ? std::min<int64_t>(f.factor_budget_mib, kFactorBudgetMiB)
                                              : kFactorBudgetMiB;
  return (size_t)mib << 20;
}

// Workspace layout, each piece 256-byte aligned: the longest-first order [N]
// (N > 1), the window table (seq_first [N+1], seq_c0 [N], seq_c1 [N]); for
// the segmented schedule the window's segment table (seg_first [N+1],
// seg_count, seg_list [2 cap]) and the affine pairs [cap][H][2][128][128]
// fp32; a state buffer [N,H,128,128] fp32 carried between windows (more than
// one window only); the factor store [slots][H] blocks.
// slots bounds the chunks of one window:
//   sum_n ceil(G_n / nw) <= (T / C + N) / nw + N,  G_n = ceil(L_n / C);
// cap bounds the segments of one window: sum_n ceil(W_n / s) <= slots / s + N
// for window ranges W_n and s chunks per segment.
struct Plan {
  int nw = 1;
  int64_t slots = 0;
  int64_t seg_chunks = 0;  // 0: sequential schedule
  int64_t cap = 0;
  size_t off_first = 0, off_c0 = 0, off_c1 = 0;
  size_t off_segfirst = 0, off_count = 0, off_list = 0, off_pairs = 0;
  size_t off_state = 0, off_factors = 0;
  size_t bytes = 0;
};

Plan make_plan(int num_seqs, int64_t total_tokens, int num_heads, kda_dtype dtype, const kda_fused_opts& f,
               int cus) {
  Plan pl;
  const bool bf = dtype == KDA_DTYPE_BF16;
  const int64_t C = kda::chunk_len(bf);
  const size_t fb = kda::factor_block_bytes(bf);
  const int64_t chunks = total_tokens / C + num_seqs;
  const double total = (double)chunks * num_heads * fb;
  pl.nw = (int)std::max<double>(1.0, std::ceil(total / (double)factor_budget(f)));
  pl.slots = chunks / pl.nw + num_seqs + 1;
  // segments are cut from each window's share of the tokens
  const int64_t seg = choose_segment_tokens(num_seqs, (total_tokens + pl.nw - 1) / pl.nw, num_heads, f, cus);
  if (seg > 0) {
    pl.seg_chunks = seg / C;
    pl.cap = pl.slots / pl.seg_chunks + num_seqs + 1;
  }
  size_t off = num_seqs > 1 ? align256((size_t)num_seqs * sizeof(int32_t)) : 0;
  pl.off_first = off;
  off += align256((size_t)(num_seqs + 1) * sizeof(int32_t));
  pl.off_c0 = off;
  off += align256((size_t)num_seqs * sizeof(int32_t));
  pl.off_c1 = off;
  off += align256((size_t)num_seqs * sizeof(int32_t));
  if (pl.seg_chunks > 0) {
    pl.off_segfirst = off;
    off += align256((size_t)(num_seqs + 1) * sizeof(int32_t));
    pl.off_count = off;
    off += 256;
    pl.off_list = off;
    off += align256((size_t)pl.cap * 2 * sizeof(int32_t));
    pl.off_pairs = off;
    off += (size_t)pl.cap * num_heads * 2 * kD * kD * sizeof(float);
  }
  pl.off_state = off;
  if (pl.nw > 1) off += (size_t)num_seqs * num_heads * kD * kD * sizeof(float);
  pl.off_factors = off;
  pl.bytes = off + (size_t)pl.slots * num_heads * fb;
  return pl;
}

const kda_fused_opts kNoOpts = {nullptr, nullptr, nullptr, nullptr, 1e-6f, 1e-6f, 0, 0, 0};
constexpr float kBoundedLaMin = -5.f;  // the K3 decay bound the tile paths rely on

// Optional precondition checks: the environment variable KDA_DEBUG_CHECKS
// (read at every call) switches them on; the failed checks of the calling
// thread's last checked call are kept for kda_last_precondition_flags().
bool debug_checks() {
  const char* e = std::getenv("KDA_DEBUG_CHECKS");
  return e && *e && std::strcmp(e, "0") != 0;
}
thread_local uint32_t t_check_flags = 0;

// Runs the checks when they are on: KDA_OK to go ahead, otherwise the status to return.
kda_status checked(const kda::CheckArgs& a, hipStream_t stream) {
  if (!debug_checks()) return KDA_OK;
  uint32_t flags = 0;
  if (kda::run_checks(a, stream, &flags) != hipSuccess) return KDA_ERR_HIP;
  t_check_flags = flags;
  return flags ? KDA_ERR_PRECONDITION : KDA_OK;
}

// The kernels address one chunk's rows of a [T, H, 128] tensor through
// buffer views with 32-bit byte offsets: 64 tokens x H x 128 x 4 bytes must
// stay below 2^31, so H is at most kMaxHeads.
constexpr int kMaxHeads = 65535;

bool sizes_ok(int num_seqs, int64_t total_tokens, int num_heads) {
  return num_seqs >= 1 && num_heads >= 1 && num_heads <= kMaxHeads && total_tokens >= 0 &&
         (int64_t)num_seqs * num_heads <= (int64_t)INT32_MAX / 2 && total_tokens <= (int64_t)INT32_MAX;
}

// A forced segment length must be a multiple of 64, and the segment list must
// fit the launch grid.
bool segments_ok(const Plan& pl, int num_heads, const kda_fused_opts& f) {
  if (f.segment_tokens > 0 && f.segment_tokens % 64 != 0) return false;
  if (f.factor_budget_mib < 0) return false;
  if (!(pl.slots <= (int64_t)INT32_MAX / 2 && pl.slots * num_heads <= (int64_t)UINT32_MAX)) return false;
  return pl.seg_chunks == 0 || pl.cap * num_heads <= (int64_t)INT32_MAX / 8;
}

// Workspace of kda_chunk_bwd: one window holding every chunk (slot = global
// chunk index).  Pieces, each 256-byte aligned: the longest-first order [N]
// (N > 1), the chunk table (seq_first [N+1], seq_c0 [N], seq_c1 [N]), the
// forward factor blocks and the reverse-carry blocks [slots][H], then per
// (slot, head) the chunk's incoming state and the gradient at its end
// ([128 x 128] each) and U and dU ([C x 128] each), in the I/O dtype as
// 16 x 16 tiles.
struct BwdPlan {
  int64_t slots = 0;
  size_t off_first = 0, off_c0 = 0, off_c1 = 0, off_factors = 0, off_dblocks = 0;
  size_t off_states = 0, off_u = 0, off_ds = 0, off_du = 0;
  size_t bytes = 0;
};

BwdPlan make_bwd_plan(int num_seqs, int64_t total_tokens, int num_heads, kda_dtype dtype) {
  BwdPlan pl;
  const bool bf = dtype == KDA_DTYPE_BF16;
  const int64_t C = kda::chunk_len(bf);
  pl.slots = total_tokens / C + num_seqs + 1;
  const size_t units = (size_t)pl.slots * num_heads;
  size_t off = num_seqs > 1 ? align256((size_t)num_seqs * sizeof(int32_t)) : 0;
  pl.off_first = off;
  off += align256((size_t)(num_seqs + 1) * sizeof(int32_t));
  pl.off_c0 = off;
  off += align256((size_t)num_seqs * sizeof(int32_t));
  pl.off_c1 = off;
  off += align256((size_t)num_seqs * sizeof(int32_t));
  pl.off_factors = off;
  off += units * kda::factor_block_bytes(bf);
  pl.off_dblocks = off;
  off += units * kda::dcarry_block_bytes(bf);
  const size_t es = bf ? 2 : 4;
  pl.off_states = off;
  off += units * kD * kD * es;
  pl.off_ds = off;
  off += units * kD * kD * es;
  pl.off_u = off;
  off += units * (size_t)C * kD * es;
  pl.off_du = off;
  off += units * (size_t)C * kD * es;
  pl.bytes = off;
  return pl;
}

bool bwd_sizes_ok(int num_seqs, int64_t total_tokens, int num_heads, kda_dtype dtype) {
  if (!sizes_ok(num_seqs, total_tokens, num_heads)) return false;
  const int64_t slots = total_tokens / kda::chunk_len(dtype == KDA_DTYPE_BF16) + num_seqs + 1;
  return slots <= (int64_t)INT32_MAX / 2 && slots * num_heads <= (int64_t)UINT32_MAX;
}

// Scratch of kda_chunk_fwd_noalloc.  Each GPU holds its own copy at its own
// address; in host code the array's name is only a stand-in, so the address
// passed to kernels is the one hipGetSymbolAddress gives for the current device.
__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "success";
    case KDA_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or illegal buffer overlap)";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration (d_k and d_v must be 128; dtype f32 or bf16)";
    case KDA_ERR_WORKSPACE: return "workspace missing or smaller than kda_chunk_fwd_workspace_bytes()";
    case KDA_ERR_HIP: return "HIP runtime or launch error";
    case KDA_ERR_PRECONDITION:
      return "input outside the documented preconditions (KDA_DEBUG_CHECKS; see kda_last_precondition_flags())";
    case KDA_ERR_SCRATCH:
      return "sizes need more device scratch than kda_chunk_fwd_noalloc holds (KDA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown kda_status";
}

uint32_t kda_last_precondition_flags(void) { return t_check_flags; }

size_t kda_chunk_fwd_workspace_bytes(int num_seqs, int64_t total_tokens, int num_heads, int d_k, int d_v,
                                     kda_dtype dtype, const kda_fused_opts* opts) {
  if (!sizes_ok(num_seqs, total_tokens, num_heads) || d_k != kD || d_v != kD || !dtype_ok(dtype)) return 0;
  const kda_fused_opts& f = opts ? *opts : kNoOpts;
  const Plan pl = make_plan(num_seqs, total_tokens, num_heads, dtype, f, cu_count_for_current_device());
  if (!segments_ok(pl, num_heads, f)) return 0;
  return pl.bytes;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                         const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                         int64_t total_tokens, int num_heads, int d_k, int d_v, kda_dtype dtype,
                         const kda_fused_opts* opts, void* o, float* final_state, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs < 1 || num_heads < 1 || total_tokens < 0) return KDA_ERR_INVALID_ARG;
  if (d_k != kD || d_v != kD || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens && num_seqs != 1) return KDA_ERR_INVALID_ARG;
  // cu_seqlens is int32; work items are counted in int32
  if (!sizes_ok(num_seqs, total_tokens, num_heads)) return KDA_ERR_INVALID_ARG;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_INVALID_ARG;
  const kda_fused_opts& f = opts ? *opts : kNoOpts;
  if (!(f.l2_eps >= 0.f) || !(f.rms_eps >= 0.f)) return KDA_ERR_INVALID_ARG;
  {
    const void* vec[] = {q, k, v, log_alpha, initial_state, o, final_state, f.gate, workspace};
    for (const void* ptr : vec)
      if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
    const void* sca[] = {beta, cu_seqlens, f.conv_q_w, f.conv_k_w, f.norm_w};
    for (const void* ptr : sca)
      if (!aligned(ptr, 4)) return KDA_ERR_INVALID_ARG;
  }

  const Plan pl = make_plan(num_seqs, total_tokens, num_heads, dtype, f, cu_count_for_current_device());
  if (!segments_ok(pl, num_heads, f)) return KDA_ERR_INVALID_ARG;
  const size_t need = pl.bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

  const size_t es = elem_size(dtype);
  const size_t tok_elems = (size_t)total_tokens * num_heads * kD;
  const size_t state_bytes = (size_t)num_seqs * num_heads * kD * kD * sizeof(float);
  const Range r_q = range_of(q, tok_elems * es), r_k = range_of(k, tok_elems * es), r_v = range_of(v, tok_elems * es);
  const Range r_la = range_of(log_alpha, tok_elems * sizeof(float));
  const Range r_b = range_of(beta, (size_t)total_tokens * num_heads * sizeof(float));
  const Range r_s0 = range_of(initial_state, state_bytes);
  const Range r_cu = range_of(cu_seqlens, cu_seqlens ? (size_t)(num_seqs + 1) * sizeof(int32_t) : 0);
  const Range r_g = range_of(f.gate, f.gate ? tok_elems * es : 0);
  const Range r_cq = range_of(f.conv_q_w, f.conv_q_w ? (size_t)num_heads * kD * 4 * sizeof(float) : 0);
  const Range r_ck = range_of(f.conv_k_w, f.conv_k_w ? (size_t)num_heads * kD * 4 * sizeof(float) : 0);
  const Range r_nw = range_of(f.norm_w, f.norm_w ? kD * sizeof(float) : 0);
  const Range r_o = range_of(o, tok_elems * es);
  const Range r_fs = range_of(final_state, final_state ? state_bytes : 0);
  const Range r_ws = range_of(workspace, need);
  // final_state may be exactly initial_state (in-place continuation); any
  // other overlap of an output with an input or another output is refused.
  const Range inputs[] = {r_q, r_k, r_v, r_la, r_b, r_s0, r_cu, r_g, r_cq, r_ck, r_nw};
  for (const Range& in : inputs) {
    if (overlap(r_o, in) || overlap(r_ws, in)) return KDA_ERR_INVALID_ARG;
    if (&in != &inputs[5] && overlap(r_fs, in)) return KDA_ERR_INVALID_ARG;
  }
  if (overlap(r_fs, r_s0) && !(r_fs.lo == r_s0.lo && r_fs.hi == r_s0.hi)) return KDA_ERR_INVALID_ARG;
  if (overlap(r_o, r_fs) || overlap(r_o, r_ws) || overlap(r_fs, r_ws)) return KDA_ERR_INVALID_ARG;

  const bool bf16 = dtype == KDA_DTYPE_BF16;
  {
    kda::CheckArgs chk;
    std::memset(&chk, 0, sizeof(chk));
    chk.rows = total_tokens * num_heads;
    chk.heads = num_heads;
    chk.tokens_per_seq = 1;
    chk.log_alpha = log_alpha;
    chk.beta = beta;
    chk.q = f.conv_q_w ? nullptr : q;
    chk.k = f.conv_k_w ? nullptr : k;
    chk.cu = cu_seqlens;
    chk.num_seqs = num_seqs;
    chk.total_tokens = total_tokens;
    chk.bf16 = bf16;
    chk.la_min = f.unbounded_decay ? -INFINITY : kBoundedLaMin;
    const kda_status cs = checked(chk, stream);
    if (cs != KDA_OK) return cs;
  }
  char* ws = static_cast<char*>(workspace);
  int32_t* order = num_seqs > 1 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + pl.off_first);
  int32_t* seq_c0 = reinterpret_cast<int32_t*>(ws + pl.off_c0);
  int32_t* seq_c1 = reinterpret_cast<int32_t*>(ws + pl.off_c1);
  float* carry_buf = final_state ? final_state : reinterpret_cast<float*>(ws + pl.off_state);
  void* factors = ws + pl.off_factors;
  const bool segmented = pl.seg_chunks > 0;
  if (num_seqs > 1 && !segmented) {
    if (kda::launch_worklist(cu_seqlens, num_seqs, order, stream) != hipSuccess) return KDA_ERR_HIP;
  }

  kda::PrepArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.log_alpha = log_alpha;
  pa.beta = beta;
  pa.cu = cu_seqlens;
  pa.conv_q_w = f.conv_q_w;
  pa.conv_k_w = f.conv_k_w;
  pa.l2_eps = f.l2_eps;
  pa.num_seqs = num_seqs;
  pa.num_heads = num_heads;
  pa.total_tokens = total_tokens;
  pa.bf16 = bf16;
  pa.seq_first = seq_first;
  pa.seq_c0 = seq_c0;
  pa.cap = (int)pl.slots;
  pa.chunks_per_block = kPrepChunksPerBlock;
  pa.factors = factors;
  pa.unbounded = f.unbounded_decay != 0;

  kda::CarryArgs ca;
  std::memset(&ca, 0, sizeof(ca));
  ca.factors = factors;
  ca.cu = cu_seqlens;
  ca.order = segmented ? nullptr : order;
  ca.seq_first = seq_first;
  ca.seq_c0 = seq_c0;
  ca.seq_c1 = seq_c1;
  ca.gate = f.gate;
  ca.norm_w = f.norm_w;
  ca.rms_eps = f.rms_eps;
  ca.o = o;
  ca.num_seqs = num_seqs;
  ca.num_heads = num_heads;
  ca.total_tokens = total_tokens;
  ca.bf16 = bf16;
  // Two value-column blocks per work item; the epilogue normalises whole
  // heads, so it keeps one.
  ca.col_split = f.gate ? 1 : 2;

  if (!segmented) {
    // Per window: the window table, the factor blocks of every (chunk, head),
    // then the state walk over them.
    ca.units = num_seqs * num_heads;
    for (int w = 0; w < pl.nw; ++w) {
      if (kda::launch_window_table(cu_seqlens, num_seqs, total_tokens, kda::chunk_len(bf16), pl.nw, w,
                                   (int)pl.slots, seq_first, seq_c0, seq_c1, stream) != hipSuccess)
        return KDA_ERR_HIP;
      if (kda::launch_prep(pa, stream) != hipSuccess) return KDA_ERR_HIP;
      ca.state_in = (w == 0) ? initial_state : carry_buf;
      ca.state_out = (w == pl.nw - 1) ? final_state : carry_buf;
      if (kda::launch_carry(ca, stream) != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
  }

  // Segmented schedule, per window: the window table and the factor blocks as
  // above; the window's segments; per segment the affine pair (B from a zero
  // state, M from the identity with V = 0); the scan over each sequence's
  // segments from the window's incoming state; then the outputs of every
  // segment from its incoming state.
  int32_t* seg_first = reinterpret_cast<int32_t*>(ws + pl.off_segfirst);
  int32_t* seg_count = reinterpret_cast<int32_t*>(ws + pl.off_count);
  int32_t* seg_list = reinterpret_cast<int32_t*>(ws + pl.off_list);
  float* pairs = reinterpret_cast<float*>(ws + pl.off_pairs);
  ca.units = (int)(pl.cap * num_heads);
  ca.seg_list = seg_list;
  ca.seg_count = seg_count;
  ca.seg_chunks = (int)pl.seg_chunks;
  ca.pairs = pairs;
  kda::CarryArgs c1 = ca;
  c1.pass = 1;
  // whole heads on two-tile waves: one B and one M workgroup per (segment,
  // head), which read the factor blocks once per 128 columns and fill the
  // GPU in one round (measured: 293-296 -> 208 us at H = 8, T = 131072,
  // against four 64-column workgroups)
  c1.col_split = 2;
  c1.gate = nullptr;
  c1.norm_w = nullptr;
  kda::CarryArgs c2 = ca;
  c2.pass = 2;
  kda::ScanArgs sc;
  sc.pairs = pairs;
  sc.seq_first = seg_first;
  sc.num_seqs = num_seqs;
  sc.num_heads = num_heads;
  for (int w = 0; w < pl.nw; ++w) {
    if (kda::launch_window_table(cu_seqlens, num_seqs, total_tokens, kda::chunk_len(bf16), pl.nw, w,
                                 (int)pl.slots, seq_first, seq_c0, seq_c1, stream) != hipSuccess)
      return KDA_ERR_HIP;
    if (kda::launch_prep(pa, stream) != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_window_segments(seq_c0, seq_c1, num_seqs, (int)pl.seg_chunks, (int)pl.cap, seg_first, seg_list,
                                    seg_count, stream) != hipSuccess)
      return KDA_ERR_HIP;
    if (kda::launch_carry(c1, stream) != hipSuccess) return KDA_ERR_HIP;
    sc.init = (w == 0) ? initial_state : carry_buf;
    sc.fin = (w == pl.nw - 1) ? final_state : carry_buf;
    if (kda::launch_scan(sc, stream) != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_carry(c2, stream) != hipSuccess) return KDA_ERR_HIP;
  }
  return KDA_OK;
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                                 int num_seqs, int64_t total_tokens, int num_heads, int d_k, int d_v,
                                 kda_dtype dtype, const kda_fused_opts* opts, void* o, float* final_state,
                                 hipStream_t stream) {
  if (num_seqs < 1 || num_heads < 1 || total_tokens < 0) return KDA_ERR_INVALID_ARG;
  if (d_k != kD || d_v != kD || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (!sizes_ok(num_seqs, total_tokens, num_heads)) return KDA_ERR_INVALID_ARG;
  const kda_fused_opts& f = opts ? *opts : kNoOpts;
  if (f.factor_budget_mib < 0) return KDA_ERR_INVALID_ARG;
  // The largest window budget whose whole plan fits the scratch array: each
  // step lowers the budget by at least the plan's excess (the plan shrinks by
  // at most that much per MiB of budget), down to 1 MiB.
  constexpr size_t kScratch = KDA_NOALLOC_SCRATCH_BYTES;
  constexpr int64_t kScratchMiB = (int64_t)(kScratch >> 20);
  int64_t mib = f.factor_budget_mib > 0 ? std::min<int64_t>(f.factor_budget_mib, kScratchMiB) : kScratchMiB;
  const int cus = cu_count_for_current_device();
  kda_fused_opts g = f;
  for (;;) {
    g.factor_budget_mib = (int)mib;
    const Plan pl = make_plan(num_seqs, total_tokens, num_heads, dtype, g, cus);
    if (!segments_ok(pl, num_heads, g)) return KDA_ERR_INVALID_ARG;
    if (pl.bytes <= kScratch) break;
    if (mib == 1) return KDA_ERR_SCRATCH;
    const int64_t over = (int64_t)((pl.bytes - kScratch + (1u << 20) - 1) >> 20);
    mib = std::max<int64_t>(1, mib - std::max<int64_t>(1, over));
  }
  void* ws = nullptr;
  if (scratch_for_current_device(&ws) != hipSuccess) return KDA_ERR_HIP;
  return kda_chunk_fwd(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, d_k,
                       d_v, dtype, &g, o, final_state, ws, kScratch, stream);
}

size_t kda_chunk_bwd_workspace_bytes(int num_seqs, int64_t total_tokens, int num_heads, int d_k, int d_v,
                                     kda_dtype dtype) {
  if (d_k != kD || d_v != kD || !dtype_ok(dtype) || !bwd_sizes_ok(num_seqs, total_tokens, num_heads, dtype)) return 0;
  return make_bwd_plan(num_seqs, total_tokens, num_heads, dtype).bytes;
}

namespace {

// Debug check of the backward's and the training forward's inputs (the
// decay bound of the plain prefill).
kda_status bwd_input_checks(const void* q, const void* k, const float* log_alpha, const float* beta,
                            const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int num_heads, bool bf16,
                            hipStream_t stream) {
  kda::CheckArgs chk;
  std::memset(&chk, 0, sizeof(chk));
  chk.rows = total_tokens * num_heads;
  chk.heads = num_heads;
  chk.tokens_per_seq = 1;
  chk.log_alpha = log_alpha;
  chk.beta = beta;
  chk.q = q;
  chk.k = k;
  chk.cu = cu_seqlens;
  chk.num_seqs = num_seqs;
  chk.total_tokens = total_tokens;
  chk.bf16 = bf16;
  chk.la_min = kBoundedLaMin;
  return checked(chk, stream);
}

// The longest-first order and the window table (one window over every
// chunk) in the backward's workspace, from cu_seqlens.
kda_status bwd_tables(const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, bool bf16, const BwdPlan& pl,
                      char* ws, hipStream_t stream) {
  int32_t* order = num_seqs > 1 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  if (num_seqs > 1 && kda::launch_worklist(cu_seqlens, num_seqs, order, stream) != hipSuccess) return KDA_ERR_HIP;
  if (kda::launch_window_table(cu_seqlens, num_seqs, total_tokens, kda::chunk_len(bf16), 1, 0, (int)pl.slots,
                               reinterpret_cast<int32_t*>(ws + pl.off_first), reinterpret_cast<int32_t*>(ws + pl.off_c0),
                               reinterpret_cast<int32_t*>(ws + pl.off_c1), stream) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

// The backward's residuals in its workspace: the tables above, the forward
// factor blocks and, per chunk, the incoming state and U (carry pass 3).
// For the training forward the same walk also writes the outputs and the
// final state (carry pass 4); o may be NULL there when there are no tokens.
kda_status bwd_residuals(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                         const float* initial_state, const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens,
                         int num_heads, bool bf16, const BwdPlan& pl, char* ws, bool forward, void* o,
                         float* final_state, hipStream_t stream) {
  const kda_status ts = bwd_tables(cu_seqlens, num_seqs, total_tokens, bf16, pl, ws, stream);
  if (ts != KDA_OK) return ts;
  int32_t* order = num_seqs > 1 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + pl.off_first);
  int32_t* seq_c0 = reinterpret_cast<int32_t*>(ws + pl.off_c0);
  int32_t* seq_c1 = reinterpret_cast<int32_t*>(ws + pl.off_c1);
  void* factors = ws + pl.off_factors;
  kda::PrepArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.log_alpha = log_alpha;
  pa.beta = beta;
  pa.cu = cu_seqlens;
  pa.l2_eps = 1e-6f;
  pa.num_seqs = num_seqs;
  pa.num_heads = num_heads;
  pa.total_tokens = total_tokens;
  pa.bf16 = bf16;
  pa.seq_first = seq_first;
  pa.seq_c0 = seq_c0;
  pa.cap = (int)pl.slots;
  pa.chunks_per_block = kPrepChunksPerBlock;
  pa.factors = factors;
  if (kda::launch_prep(pa, stream) != hipSuccess) return KDA_ERR_HIP;
  kda::CarryArgs ca;
  std::memset(&ca, 0, sizeof(ca));
  ca.factors = factors;
  ca.cu = cu_seqlens;
  ca.order = order;
  ca.seq_first = seq_first;
  ca.seq_c0 = seq_c0;
  ca.seq_c1 = seq_c1;
  ca.state_in = initial_state;
  ca.state_out = forward ? final_state : nullptr;
  ca.o = o;
  ca.rms_eps = 1e-6f;
  ca.num_seqs = num_seqs;
  ca.num_heads = num_heads;
  ca.total_tokens = total_tokens;
  ca.units = num_seqs * num_heads;
  ca.col_split = 2;
  ca.bf16 = bf16;
  ca.pass = forward ? 4 : 3;
  ca.chunk_states = ws + pl.off_states;
  ca.chunk_u = ws + pl.off_u;
  if (kda::launch_carry(ca, stream) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

// The gradients from the residuals: reverse-carry blocks, the reverse carry,
// the per-chunk gradients.
kda_status bwd_gradients(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                         const int32_t* cu_seqlens, const void* d_o, const float* d_final_state, int num_seqs,
                         int64_t total_tokens, int num_heads, bool bf16, const BwdPlan& pl, char* ws, void* dq,
                         void* dk, void* dv, float* dlog_alpha, float* dbeta, float* d_initial_state,
                         hipStream_t stream) {
  kda::BwdArgs ba;
  std::memset(&ba, 0, sizeof(ba));
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.log_alpha = log_alpha;
  ba.beta = beta;
  ba.d_o = d_o;
  ba.d_final_state = d_final_state;
  ba.cu = cu_seqlens;
  ba.order = num_seqs > 1 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  ba.seq_first = reinterpret_cast<int32_t*>(ws + pl.off_first);
  ba.num_seqs = num_seqs;
  ba.num_heads = num_heads;
  ba.total_tokens = total_tokens;
  ba.slots = (int)pl.slots;
  ba.bf16 = bf16;
  ba.factors = ws + pl.off_factors;
  ba.dblocks = ws + pl.off_dblocks;
  ba.chunk_states = ws + pl.off_states;
  ba.chunk_u = ws + pl.off_u;
  ba.chunk_ds = ws + pl.off_ds;
  ba.chunk_du = ws + pl.off_du;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.dlog_alpha = dlog_alpha;
  ba.dbeta = dbeta;
  ba.d_initial_state = d_initial_state;
  if (kda::launch_bwd_prep(ba, stream) != hipSuccess) return KDA_ERR_HIP;
  if (kda::launch_bwd_carry(ba, stream) != hipSuccess) return KDA_ERR_HIP;
  if (kda::launch_bwd_grad(ba, stream) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

// Argument checks of kda_chunk_bwd and kda_chunk_bwd_saved.
kda_status bwd_args_ok(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                       const float* initial_state, const int32_t* cu_seqlens, const void* d_o,
                       const float* d_final_state, int num_seqs, int64_t total_tokens, int num_heads, int d_k,
                       int d_v, kda_dtype dtype, const void* dq, const void* dk, const void* dv,
                       const float* dlog_alpha, const float* dbeta, const float* d_initial_state,
                       const void* workspace, size_t workspace_bytes) {
  if (num_seqs < 1 || num_heads < 1 || total_tokens < 0) return KDA_ERR_INVALID_ARG;
  if (d_k != kD || d_v != kD || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens && num_seqs != 1) return KDA_ERR_INVALID_ARG;
  if (!bwd_sizes_ok(num_seqs, total_tokens, num_heads, dtype)) return KDA_ERR_INVALID_ARG;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !dq || !dk || !dv || !dlog_alpha ||
                           !dbeta))
    return KDA_ERR_INVALID_ARG;
  {
    const void* vec[] = {q, k, v, log_alpha, initial_state, d_o, d_final_state, dq, dk, dv, dlog_alpha,
                         d_initial_state, workspace};
    for (const void* ptr : vec)
      if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
    const void* sca[] = {beta, cu_seqlens, dbeta};
    for (const void* ptr : sca)
      if (!aligned(ptr, 4)) return KDA_ERR_INVALID_ARG;
  }
  const BwdPlan pl = make_bwd_plan(num_seqs, total_tokens, num_heads, dtype);
  if (!workspace || workspace_bytes < pl.bytes) return KDA_ERR_WORKSPACE;

  const size_t es = elem_size(dtype);
  const size_t tok_elems = (size_t)total_tokens * num_heads * kD;
  const size_t state_bytes = (size_t)num_seqs * num_heads * kD * kD * sizeof(float);
  const size_t beta_bytes = (size_t)total_tokens * num_heads * sizeof(float);
  const Range ins[] = {range_of(q, tok_elems * es), range_of(k, tok_elems * es), range_of(v, tok_elems * es),
                       range_of(log_alpha, tok_elems * sizeof(float)), range_of(beta, beta_bytes),
                       range_of(initial_state, state_bytes),
                       range_of(cu_seqlens, cu_seqlens ? (size_t)(num_seqs + 1) * sizeof(int32_t) : 0),
                       range_of(d_o, tok_elems * es), range_of(d_final_state, d_final_state ? state_bytes : 0)};
  const Range outs[] = {range_of(dq, tok_elems * es), range_of(dk, tok_elems * es), range_of(dv, tok_elems * es),
                        range_of(dlog_alpha, tok_elems * sizeof(float)), range_of(dbeta, beta_bytes),
                        range_of(d_initial_state, d_initial_state ? state_bytes : 0),
                        range_of(workspace, pl.bytes)};
  constexpr int kOuts = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < kOuts; ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return KDA_ERR_INVALID_ARG;
    for (int j = i + 1; j < kOuts; ++j)
      if (overlap(outs[i], outs[j])) return KDA_ERR_INVALID_ARG;
  }
  return KDA_OK;
}

}  // namespace

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                         const float* initial_state, const int32_t* cu_seqlens, const void* d_o,
                         const float* d_final_state, int num_seqs, int64_t total_tokens, int num_heads, int d_k,
                         int d_v, kda_dtype dtype, void* dq, void* dk, void* dv, float* dlog_alpha, float* dbeta,
                         float* d_initial_state, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const kda_status st = bwd_args_ok(q, k, v, log_alpha, beta, initial_state, cu_seqlens, d_o, d_final_state,
                                    num_seqs, total_tokens, num_heads, d_k, d_v, dtype, dq, dk, dv, dlog_alpha, dbeta,
                                    d_initial_state, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  const bool bf16 = dtype == KDA_DTYPE_BF16;
  const kda_status cs = bwd_input_checks(q, k, log_alpha, beta, cu_seqlens, num_seqs, total_tokens, num_heads, bf16,
                                         stream);
  if (cs != KDA_OK) return cs;
  const BwdPlan pl = make_bwd_plan(num_seqs, total_tokens, num_heads, dtype);
  char* ws = static_cast<char*>(workspace);
  const kda_status rs = bwd_residuals(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, total_tokens,
                                      num_heads, bf16, pl, ws, false, nullptr, nullptr, stream);
  if (rs != KDA_OK) return rs;
  return bwd_gradients(q, k, v, log_alpha, beta, cu_seqlens, d_o, d_final_state, num_seqs, total_tokens, num_heads,
                       bf16, pl, ws, dq, dk, dv, dlog_alpha, dbeta, d_initial_state, stream);
}

kda_status kda_chunk_fwd_save(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                              int64_t total_tokens, int num_heads, int d_k, int d_v, kda_dtype dtype, void* o,
                              float* final_state, void* bwd_workspace, size_t bwd_workspace_bytes,
                              hipStream_t stream) {
  if (num_seqs < 1 || num_heads < 1 || total_tokens < 0) return KDA_ERR_INVALID_ARG;
  if (d_k != kD || d_v != kD || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens && num_seqs != 1) return KDA_ERR_INVALID_ARG;
  if (!bwd_sizes_ok(num_seqs, total_tokens, num_heads, dtype)) return KDA_ERR_INVALID_ARG;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_INVALID_ARG;
  {
    const void* vec[] = {q, k, v, log_alpha, initial_state, o, final_state, bwd_workspace};
    for (const void* ptr : vec)
      if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
    const void* sca[] = {beta, cu_seqlens};
    for (const void* ptr : sca)
      if (!aligned(ptr, 4)) return KDA_ERR_INVALID_ARG;
  }
  const BwdPlan pl = make_bwd_plan(num_seqs, total_tokens, num_heads, dtype);
  if (!bwd_workspace || bwd_workspace_bytes < pl.bytes) return KDA_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t tok_elems = (size_t)total_tokens * num_heads * kD;
  const size_t state_bytes = (size_t)num_seqs * num_heads * kD * kD * sizeof(float);
  const Range r_s0 = range_of(initial_state, state_bytes);
  const Range ins[] = {range_of(q, tok_elems * es), range_of(k, tok_elems * es), range_of(v, tok_elems * es),
                       range_of(log_alpha, tok_elems * sizeof(float)),
                       range_of(beta, (size_t)total_tokens * num_heads * sizeof(float)), r_s0,
                       range_of(cu_seqlens, cu_seqlens ? (size_t)(num_seqs + 1) * sizeof(int32_t) : 0)};
  const Range r_o = range_of(o, tok_elems * es), r_fs = range_of(final_state, final_state ? state_bytes : 0),
              r_ws = range_of(bwd_workspace, pl.bytes);
  for (const Range& in : ins) {
    if (overlap(r_o, in) || overlap(r_ws, in)) return KDA_ERR_INVALID_ARG;
    if (&in != &ins[5] && overlap(r_fs, in)) return KDA_ERR_INVALID_ARG;
  }
  // final_state may be exactly initial_state (in-place continuation)
  if (overlap(r_fs, r_s0) && !(r_fs.lo == r_s0.lo && r_fs.hi == r_s0.hi)) return KDA_ERR_INVALID_ARG;
  if (overlap(r_o, r_fs) || overlap(r_o, r_ws) || overlap(r_fs, r_ws)) return KDA_ERR_INVALID_ARG;
  const bool bf16 = dtype == KDA_DTYPE_BF16;
  const kda_status cs = bwd_input_checks(q, k, log_alpha, beta, cu_seqlens, num_seqs, total_tokens, num_heads, bf16,
                                         stream);
  if (cs != KDA_OK) return cs;
  return bwd_residuals(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, bf16,
                       pl, static_cast<char*>(bwd_workspace), true, o, final_state, stream);
}

kda_status kda_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                               const void* d_o, const float* d_final_state, int num_seqs, int64_t total_tokens,
                               int num_heads, int d_k, int d_v, kda_dtype dtype, void* dq, void* dk, void* dv,
                               float* dlog_alpha, float* dbeta, float* d_initial_state, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  const kda_status st = bwd_args_ok(q, k, v, log_alpha, beta, initial_state, cu_seqlens, d_o, d_final_state,
                                    num_seqs, total_tokens, num_heads, d_k, d_v, dtype, dq, dk, dv, dlog_alpha, dbeta,
                                    d_initial_state, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  const bool bf16 = dtype == KDA_DTYPE_BF16;
  const kda_status cs = bwd_input_checks(q, k, log_alpha, beta, cu_seqlens, num_seqs, total_tokens, num_heads, bf16,
                                         stream);
  if (cs != KDA_OK) return cs;
  // the tables again, from this call's cu_seqlens: the same values for the
  // forward's inputs, and every slot index within this plan whatever it holds
  const BwdPlan pl = make_bwd_plan(num_seqs, total_tokens, num_heads, dtype);
  char* ws = static_cast<char*>(workspace);
  const kda_status ts = bwd_tables(cu_seqlens, num_seqs, total_tokens, bf16, pl, ws, stream);
  if (ts != KDA_OK) return ts;
  return bwd_gradients(q, k, v, log_alpha, beta, cu_seqlens, d_o, d_final_state, num_seqs, total_tokens, num_heads,
                       bf16, pl, ws, dq, dk, dv, dlog_alpha, dbeta, d_initial_state, stream);
}

kda_status kda_decode_step(float* state, const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, int num_seqs, int num_heads, int d_k, int d_v, kda_dtype dtype,
                           void* o, hipStream_t stream) {
  if (num_seqs < 1 || num_heads < 1) return KDA_ERR_INVALID_ARG;
  if (d_k != kD || d_v != kD || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (!state || !q || !k || !v || !log_alpha || !beta || !o) return KDA_ERR_INVALID_ARG;
  {
    if (!aligned(state, 16)) return KDA_ERR_INVALID_ARG;
    const void* sca[] = {q, k, v, log_alpha, beta, o};
    for (const void* ptr : sca)
      if (!aligned(ptr, dtype == KDA_DTYPE_BF16 ? 2 : 4)) return KDA_ERR_INVALID_ARG;
  }
  const int64_t units = (int64_t)num_seqs * num_heads;
  if (units > (int64_t)INT32_MAX) return KDA_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  const Range r_s = range_of(state, (size_t)units * kD * kD * sizeof(float));
  const Range r_q = range_of(q, (size_t)units * kD * es), r_k = range_of(k, (size_t)units * kD * es),
              r_v = range_of(v, (size_t)units * kD * es);
  const Range r_la = range_of(log_alpha, (size_t)units * kD * sizeof(float));
  const Range r_b = range_of(beta, (size_t)units * sizeof(float));
  const Range r_o = range_of(o, (size_t)units * kD * es);
  const Range inputs[] = {r_q, r_k, r_v, r_la, r_b};
  for (const Range& in : inputs)
    if (overlap(r_o, in) || overlap(r_s, in)) return KDA_ERR_INVALID_ARG;
  if (overlap(r_o, r_s)) return KDA_ERR_INVALID_ARG;
  {
    kda::CheckArgs chk;
    std::memset(&chk, 0, sizeof(chk));
    chk.rows = units;
    chk.heads = num_heads;
    chk.tokens_per_seq = 1;
    chk.log_alpha = log_alpha;
    chk.beta = beta;
    chk.q = q;
    chk.k = k;
    chk.bf16 = dtype == KDA_DTYPE_BF16;
    chk.la_min = -INFINITY;  // one token at a time: no bound needed
    const kda_status cs = checked(chk, stream);
    if (cs != KDA_OK) return cs;
  }

  kda::DecodeArgs a;
  a.state = state;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.o = o;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.bf16 = (dtype == KDA_DTYPE_BF16);
  if (kda::launch_decode(a, stream) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status kda_decode_replay(const float* state_in, float* state_out, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const int32_t* num_tokens, int num_seqs,
                             int max_tokens, int num_heads, int d_k, int d_v, kda_dtype dtype,
                             const kda_fused_opts* opts, void* conv_q_state, void* conv_k_state, void* o,
                             hipStream_t stream) {
  if (num_seqs < 1 || num_heads < 1 || max_tokens < 1) return KDA_ERR_INVALID_ARG;
  if (d_k != kD || d_v != kD || !dtype_ok(dtype) || max_tokens > kda::kReplayMaxTokens) return KDA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !log_alpha || !beta) return KDA_ERR_INVALID_ARG;
  const kda_fused_opts& f = opts ? *opts : kNoOpts;
  if (!(f.l2_eps >= 0.f) || !(f.rms_eps >= 0.f)) return KDA_ERR_INVALID_ARG;
  if ((f.conv_q_w && !conv_q_state) || (f.conv_k_w && !conv_k_state)) return KDA_ERR_INVALID_ARG;
  // a history without its convolution is neither read nor written
  if (!f.conv_q_w) conv_q_state = nullptr;
  if (!f.conv_k_w) conv_k_state = nullptr;
  {
    const void* vec[] = {state_in, state_out, q, k, v, log_alpha, f.gate, o, conv_q_state, conv_k_state};
    for (const void* ptr : vec)
      if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
    const void* sca[] = {beta, num_tokens, f.conv_q_w, f.conv_k_w, f.norm_w};
    for (const void* ptr : sca)
      if (!aligned(ptr, 4)) return KDA_ERR_INVALID_ARG;
  }
  const int64_t units = (int64_t)num_seqs * num_heads;
  if (units > (int64_t)INT32_MAX || units * max_tokens > (int64_t)INT32_MAX) return KDA_ERR_INVALID_ARG;
  if (!o && !state_out) return KDA_OK;  // nothing to produce

  const size_t es = elem_size(dtype);
  const size_t tok_elems = (size_t)units * max_tokens * kD;
  const size_t state_bytes = (size_t)units * kD * kD * sizeof(float);
  const size_t hist_bytes = (size_t)units * 3 * kD * es;
  const Range r_s0 = range_of(state_in, state_bytes), r_s1 = range_of(state_out, state_bytes);
  const Range r_q = range_of(q, tok_elems * es), r_k = range_of(k, tok_elems * es), r_v = range_of(v, tok_elems * es);
  const Range r_la = range_of(log_alpha, tok_elems * sizeof(float));
  const Range r_b = range_of(beta, (size_t)units * max_tokens * sizeof(float));
  const Range r_nt = range_of(num_tokens, num_tokens ? (size_t)num_seqs * sizeof(int32_t) : 0);
  const Range r_g = range_of(f.gate, f.gate ? tok_elems * es : 0);
  const Range r_cq = range_of(f.conv_q_w, f.conv_q_w ? (size_t)num_heads * kD * 4 * sizeof(float) : 0);
  const Range r_ck = range_of(f.conv_k_w, f.conv_k_w ? (size_t)num_heads * kD * 4 * sizeof(float) : 0);
  const Range r_nw = range_of(f.norm_w, f.norm_w ? kD * sizeof(float) : 0);
  const Range r_hq = range_of(conv_q_state, conv_q_state ? hist_bytes : 0);
  const Range r_hk = range_of(conv_k_state, conv_k_state ? hist_bytes : 0);
  const Range r_o = range_of(o, o ? tok_elems * es : 0);
  // state_out may be exactly state_in (in place); any other overlap of an
  // output with an input or another output is refused.
  const Range inputs[] = {r_s0, r_q, r_k, r_v, r_la, r_b, r_nt, r_g, r_cq, r_ck, r_nw};
  for (const Range& in : inputs) {
    if (overlap(r_o, in) || overlap(r_hq, in) || overlap(r_hk, in)) return KDA_ERR_INVALID_ARG;
    if (&in != &inputs[0] && overlap(r_s1, in)) return KDA_ERR_INVALID_ARG;
  }
  if (overlap(r_s1, r_s0) && !(r_s1.lo == r_s0.lo && r_s1.hi == r_s0.hi)) return KDA_ERR_INVALID_ARG;
  if (overlap(r_o, r_s1) || overlap(r_o, r_hq) || overlap(r_o, r_hk) || overlap(r_s1, r_hq) ||
      overlap(r_s1, r_hk) || overlap(r_hq, r_hk))
    return KDA_ERR_INVALID_ARG;
  {
    kda::CheckArgs chk;
    std::memset(&chk, 0, sizeof(chk));
    chk.rows = units * max_tokens;
    chk.heads = num_heads;
    chk.tokens_per_seq = max_tokens;
    chk.counts = num_tokens;
    chk.log_alpha = log_alpha;
    chk.beta = beta;
    chk.q = f.conv_q_w ? nullptr : q;
    chk.k = f.conv_k_w ? nullptr : k;
    chk.bf16 = dtype == KDA_DTYPE_BF16;
    chk.la_min = f.unbounded_decay ? -INFINITY : kBoundedLaMin;
    const kda_status cs = checked(chk, stream);
    if (cs != KDA_OK) return cs;
  }

  kda::ReplayArgs a;
  std::memset(&a, 0, sizeof(a));
  a.state_in = state_in;
  a.state_out = state_out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.num_tokens = num_tokens;
  a.conv_q_w = f.conv_q_w;
  a.conv_k_w = f.conv_k_w;
  a.conv_q_state = conv_q_state;
  a.conv_k_state = conv_k_state;
  a.gate = f.gate;
  a.norm_w = f.norm_w;
  a.l2_eps = f.l2_eps;
  a.rms_eps = f.rms_eps;
  a.o = o;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.max_tokens = max_tokens;
  a.bf16 = (dtype == KDA_DTYPE_BF16);
  a.unbounded = f.unbounded_decay != 0;
  if (kda::launch_replay(a, stream) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"
