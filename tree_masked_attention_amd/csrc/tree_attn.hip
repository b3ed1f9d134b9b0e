// C ABI of libtreeattn.so: argument checks, launch planning, launches.
//
// Every check that can fail runs before the first HIP call, so an error
// status means nothing was launched.  The library owns no device memory.
#include "tree_attn.h"
#ifdef TREE_ATTN_DEBUG
#include "tree_attn_debug.h"
#endif

#include <atomic>
#include <cmath>
#include <mutex>
#include <tuple>

#include "accept_commit.hpp"
#include "attn_fwd.hpp"
#include "attn_fwd128h.hpp"
#include "attn_fwd8.hpp"
#include "attn_merge.hpp"
#include "common.hpp"
#include "gdn.hpp"
#include "mask_build.hpp"
#include "tree_build.hpp"

using namespace tree_attn;

// Device scratch of tree_attn_verify_noalloc (see device_scratch below).
static __device__ __align__(256) unsigned char
    scratch[TREE_ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kAbiVersion = 11;
constexpr int kMaxDevices = 64;
constexpr int kMaxSplits = 256;
constexpr int kMinKeysPerSplit = 256;
// launches of up to this many sequences balance their splits on the device
// (one lane per sequence in split_plan.hpp)
constexpr int kBalancedMaxSeqs = 64;
// keys per workgroup from which the 256-row kernel (8 waves of 32 rows) is
// used; shorter key ranges take the 128-row kernel (8 waves: 4 row groups
// x 2 key halves).  Both kernels run 8 waves per workgroup.
constexpr int kMinKeysPerWG8 = 2048;
constexpr int kWaves = 8;
constexpr int kMaxTokenBytes = 1 << 20;

std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (queried once per device).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    return 256;
  }
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      n <= 0) {
    n = 256;
  }
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Launches a kernel on stream st and returns that launch's own status
// (hipLaunchKernel's return code).  An error that an earlier, unrelated HIP
// call left pending on this thread is neither reported nor cleared.
template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
           const Args&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel arguments");
  std::tuple<KArgs...> vals(args...);
  void* ptrs[sizeof...(KArgs)];
  std::apply(
      [&ptrs](auto&... v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
      },
      vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                         ptrs, 0, st) == hipSuccess
             ? TREE_ATTN_OK
             : TREE_ATTN_ERR_HIP;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int rows = 128;    // query rows per workgroup (64: 4 waves; 128, 256: 8)
  bool uniform = false;  // keep the host's uniform unit plan (no balancing)
  int mblocks = 0;   // row blocks per (sequence, kv head)
  int splits = 1;    // key-range splits
  int chunk = 0;     // keys per split (multiple of the 64-key tile)
  int units = 0;     // sequences * kv heads * splits * row blocks
  int blocks = 0;    // sequences * kv heads * row blocks (merge counters)
  int max_chunk = 0; // longest split whose page ids fit the kernels' LDS
  size_t part_ml_off = 0;
  size_t ws_bytes = 0;
};

// Workspace of a split launch (both paths, so that one workspace can serve
// both): kCounterBytes of arrival counters, then the fp16 partials
// [splits][N*Hq][D], then the (max, row sum) pairs [splits][N*Hq][2].
// The counter area sits at a fixed offset whatever the sizes, so counters
// left at zero by one call are zero for the next call of any shape.
size_t partials_bytes(size_t rows_all, int D, size_t* part_ml_off) {
  *part_ml_off = kCounterBytes + align_up(rows_all * D * sizeof(_Float16), 256);
  return *part_ml_off + align_up(rows_all * 2 * sizeof(float), 256);
}

// Launch planning from host-side bounds only (no device-to-host copy).
// Row blocks: 256 rows (8 waves of 32 rows) when a (sequence, kv head)
// pair has at least 256 rows and a workgroup gets a long key range, else
// 128 rows (8 waves: 4 row groups x 2 key halves), or 64 rows (4 waves)
// for pairs of at most 64 rows and for bandwidth-bound launches in which
// 64-row blocks fill the CUs without a split; any shape takes a CU's LDS.  The key range [0, max_prefix_len + max_nodes) is cut into
// splits so that the grid offers about one workgroup per CU, with at least
// 256 keys per split, and each split's page-table slice fits the kernel's
// LDS page cache.
int make_plan(int S, int N, int Hq, int Hkv, int max_prefix_len,
              int max_nodes, int page_size, int req_splits, int cus,
              Plan* out, int head_dim = kHeadDim,
              int row_bytes = kHeadDim * 2) {
  Plan pl;
  const int G = Hq / Hkv;
  const long long rows = (long long)G * max_nodes;
  const long long T = std::max(1LL, (long long)max_prefix_len + max_nodes);
  const long long max_chunk =
      std::max<long long>(kKeyTile, ((long long)(kPageCache - 1) * page_size) /
                                        kKeyTile * kKeyTile);
  const long long min_splits = (T + max_chunk - 1) / max_chunk;
  // Splits of the key range so that the work units fill the CUs (or the
  // requested count), each a whole number of 64-key tiles.
  long long splits = 0, chunk = 0, units0 = 0;
  auto choose = [&](int rows_per_wg) -> int {
    pl.rows = rows_per_wg;
    pl.mblocks = (int)std::max(1LL, (rows + rows_per_wg - 1) / rows_per_wg);
    units0 = (long long)S * Hkv * pl.mblocks;
    if (req_splits > 0) {
      splits = req_splits;
    } else {
      splits = (cus + units0 - 1) / std::max(1LL, units0);
      splits = std::min(splits, std::max(1LL, T / kMinKeysPerSplit));
    }
    splits = std::max(std::max(1LL, splits), min_splits);
    if (splits > kMaxSplits) {
      if (min_splits > kMaxSplits) return TREE_ATTN_ERR_UNSUPPORTED;
      splits = kMaxSplits;
    }
    chunk = (T + splits - 1) / splits;
    chunk = (chunk + kKeyTile - 1) / kKeyTile * kKeyTile;
    chunk = std::min(chunk, max_chunk);
    splits = (T + chunk - 1) / chunk;
    return TREE_ATTN_OK;
  };
  // 256 rows per workgroup (each staged K/V tile serves twice the rows)
  // pays off on long key ranges per workgroup; it needs 256 rows and the
  // ancestor-mask words of such a block (at most 256/G + 1 nodes) in the
  // kernel's LDS cache.  Else 128 rows (at most 129 nodes x 16 words,
  // which always fits).
  const long long mask_words = (max_nodes + 63) / 64;
  const long long nodes8 = (kRowsPerWG8 + G - 1) / G + 1;
  const bool can8 = rows >= kRowsPerWG8 && nodes8 * mask_words <= kMaskCache;
  int rpw = kRowsPerWG128;
  if (can8) {
    const int st = choose(kRowsPerWG8);
    if (st != TREE_ATTN_OK) return st;
    if (chunk >= kMinKeysPerWG8) rpw = kRowsPerWG8;
  }
  {
    const int st = choose(rpw);
    if (st != TREE_ATTN_OK) return st;
  }
  // Bandwidth-bound launches whose (sequence, kv head) pairs have at most
  // 128 rows: when 64-row blocks alone give every CU a workgroup, they
  // replace a split of the key range (the two blocks of a pair read the
  // same K/V, which the XCD-aware order keeps in one L2), so no partials
  // are written or merged.  Only for cached rows of 256 bytes (bf16, head
  // dim 128): with narrower rows (fp8, or head dim 64) a tile moves half
  // the bytes or less for the same vector work (fp8: the conversions too),
  // and the 64-row kernel's single wave per SIMD costs more than the split.
  // Those launches keep the split on 128-row blocks with the host's
  // uniform plan: the device-balanced plan reads every sequence's bounds
  // before a workgroup knows its unit, a memory round trip ahead of its
  // page-table slice (measured ~2.5 us per launch on the 30B shape, more
  // than balancing gains there).
  if (rpw == kRowsPerWG128 && req_splits <= 0 && rows <= kRowsPerWG128 &&
      splits > 1 && min_splits == 1) {
    const long long units64 =
        (long long)S * Hkv * ((rows + kRowsPerWG64 - 1) / kRowsPerWG64);
    if (units64 >= cus) {
      if (row_bytes == kHeadDim * 2) {
        const int st = choose(kRowsPerWG64);
        if (st != TREE_ATTN_OK) return st;
      } else {
        pl.uniform = true;
      }
    }
  }
  // Pairs of at most 64 rows: a 128-row block would run half its waves on
  // rows that do not exist, so 64-row blocks take them (with or without a
  // split of the key range).
  if (rpw == kRowsPerWG128 && rows <= kRowsPerWG64) {
    const int st = choose(kRowsPerWG64);
    if (st != TREE_ATTN_OK) return st;
  }
  pl.splits = (int)splits;
  pl.chunk = (int)chunk;
  pl.max_chunk = (int)max_chunk;
  const long long units = units0 * splits;
  if (units > (1LL << 30)) return TREE_ATTN_ERR_UNSUPPORTED;
  pl.units = (int)units;
  pl.blocks = (int)units0;
  if (splits > 1) {
    // one slot of partial rows per unit (split_plan.hpp)
    pl.ws_bytes = partials_bytes((size_t)pl.units * pl.rows, head_dim,
                                 &pl.part_ml_off);
  }
  *out = pl;
  return TREE_ATTN_OK;
}

int check_sizes(int S, int N, int Hq, int Hkv, int head_dim,
                int max_prefix_len, int max_nodes) {
  if (S < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || head_dim <= 0 ||
      max_prefix_len < 0 || max_nodes < 0) {
    return TREE_ATTN_ERR_SHAPE;
  }
  if (Hq % Hkv != 0) return TREE_ATTN_ERR_SHAPE;
  if (head_dim != kHeadDim) return TREE_ATTN_ERR_UNSUPPORTED;
  if (max_nodes > TREE_ATTN_MAX_NODES) return TREE_ATTN_ERR_UNSUPPORTED;
  if ((long long)max_prefix_len + max_nodes > (1LL << 30)) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  return TREE_ATTN_OK;
}

int check_accept(const int32_t* parents, const int32_t* tree_offsets,
                 const uint64_t* masks, int mask_words,
                 const int32_t* draft_tokens, const int32_t* target_tokens,
                 const int32_t* root_tokens, int num_seqs, int total_nodes,
                 int max_nodes, const int32_t* accept_len,
                 const int32_t* accept_nodes, const int32_t* bonus_tokens) {
  if (num_seqs < 0 || total_nodes < 0 || max_nodes < 0 || mask_words < 1) {
    return TREE_ATTN_ERR_SHAPE;
  }
  if (mask_words > kAcceptMaxWords || max_nodes > TREE_ATTN_MAX_NODES) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if ((long long)mask_words * 64 < max_nodes) return TREE_ATTN_ERR_SHAPE;
  if (num_seqs == 0) return TREE_ATTN_OK;
  if (!tree_offsets || !root_tokens || !accept_len || !bonus_tokens) {
    return TREE_ATTN_ERR_NULL;
  }
  if (max_nodes > 0 && !accept_nodes) return TREE_ATTN_ERR_NULL;
  if (total_nodes > 0 &&
      (!parents || !masks || !draft_tokens || !target_tokens)) {
    return TREE_ATTN_ERR_NULL;
  }
  return TREE_ATTN_OK;
}

AcceptArgs accept_args(const int32_t* parents, const int32_t* tree_offsets,
                       const uint64_t* masks, int mask_words,
                       const int32_t* draft_tokens,
                       const int32_t* target_tokens,
                       const int32_t* root_tokens, int total_nodes,
                       int max_nodes, int32_t* accept_len,
                       int32_t* accept_nodes, int32_t* bonus_tokens) {
  AcceptArgs ap;
  ap.parents = parents;
  ap.offsets = tree_offsets;
  ap.masks = masks;
  ap.draft = draft_tokens;
  ap.target = target_tokens;
  ap.root_tokens = root_tokens;
  ap.accept_len = accept_len;
  ap.accept_nodes = accept_nodes;
  ap.bonus = bonus_tokens;
  ap.W = mask_words;
  ap.total_nodes = total_nodes;
  ap.max_nodes = max_nodes;
  return ap;
}

// Checks of the cache arguments of a commit (the accepted lists are
// checked by the caller: the fused call writes them itself).
int check_commit(const void* k_cache, const void* v_cache,
                 const int32_t* page_table, int max_pages_per_seq,
                 int num_pages, int page_size, const int32_t* prefix_lens,
                 int num_seqs, int max_nodes, int token_bytes) {
  if (num_seqs < 0 || max_nodes < 0 || max_pages_per_seq < 0 ||
      num_pages < 0 || token_bytes <= 0 || token_bytes % 16 != 0 ||
      !is_pow2(page_size)) {
    return TREE_ATTN_ERR_SHAPE;
  }
  if (max_nodes > TREE_ATTN_MAX_NODES || token_bytes > kMaxTokenBytes) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0 || max_nodes == 0) return TREE_ATTN_OK;
  if (!k_cache || !v_cache || !page_table || !prefix_lens) {
    return TREE_ATTN_ERR_NULL;
  }
  if ((reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0) {
    return TREE_ATTN_ERR_SHAPE;
  }
  return TREE_ATTN_OK;
}

CommitParams commit_params(void* k_cache, void* v_cache,
                           const int32_t* page_table, int max_pages_per_seq,
                           int num_pages, int page_size,
                           const int32_t* prefix_lens,
                           const int32_t* accept_len,
                           const int32_t* accept_nodes, int max_nodes,
                           int token_bytes, int threads) {
  CommitParams cp;
  cp.k = static_cast<uint8_t*>(k_cache);
  cp.v = static_cast<uint8_t*>(v_cache);
  cp.page_table = page_table;
  cp.prefix_lens = prefix_lens;
  cp.accept_len = accept_len;
  cp.accept_nodes = accept_nodes;
  cp.max_pages = max_pages_per_seq;
  cp.num_pages = num_pages;
  cp.log2_page = ilog2(page_size);
  cp.max_nodes = max_nodes;
  cp.pieces = token_bytes / 16;
  cp.slices = (2 * cp.pieces + threads - 1) / threads;
  cp.token_bytes = token_bytes;
  return cp;
}

// Size checks of a verify call (everything but the pointers).
int check_verify_sizes(int S, int N, int Hq, int Hkv, int head_dim,
                       int max_prefix_len, int max_nodes, int num_splits,
                       int mask_words, int max_pages_per_seq, int num_pages,
                       int page_size, float scale) {
  int st = check_sizes(S, N, Hq, Hkv, head_dim, max_prefix_len, max_nodes);
  if (st != TREE_ATTN_OK) return st;
  if (num_splits < 0 || mask_words < 1 || max_pages_per_seq < 0 ||
      num_pages < 0) {
    return TREE_ATTN_ERR_SHAPE;
  }
  if (!is_pow2(page_size) || page_size > 4096) return TREE_ATTN_ERR_SHAPE;
  if ((long long)mask_words * 64 < max_nodes) return TREE_ATTN_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return TREE_ATTN_ERR_SHAPE;
  if (S == 0 || N == 0) return TREE_ATTN_OK;
  if (num_pages < 1 || max_pages_per_seq < 1) return TREE_ATTN_ERR_SHAPE;
  return TREE_ATTN_OK;
}

// The device-side unit plan of a launch (split_plan.hpp).  Launches that
// split the key range and hold 2 .. 64 sequences are balanced on the
// device from the actual sequence lengths; one sequence, forced splits,
// unsplit launches and larger batches use the host's uniform plan.
SplitParams split_params(const Plan& pl, const int32_t* prefix_lens,
                         const int32_t* tree_offsets, int S, int N, int Hkv,
                         int G, int max_tokens, int max_prefix_len,
                         int max_nodes, int req_splits) {
  SplitParams q;
  q.prefix_lens = prefix_lens;
  q.tree_offsets = tree_offsets;
  q.S = S;
  q.N = N;
  q.Hkv = Hkv;
  q.G = G;
  q.rows_per_wg = pl.rows;
  q.max_tokens = (int)std::min<long long>(
      max_tokens, (long long)max_prefix_len + max_nodes);
  q.max_nodes = max_nodes;
  q.parts = pl.units;
  q.chunk_max = pl.max_chunk;
  q.chunk_min = std::min(kMinKeysPerSplit, pl.max_chunk);
  const bool balanced = req_splits <= 0 && pl.splits > 1 && S > 1 &&
                        S <= kBalancedMaxSeqs && !pl.uniform;
  q.uniform_chunk = balanced ? 0 : pl.chunk;
  q.uniform_splits = pl.splits;
  q.uniform_mblocks = pl.mblocks;
  return q;
}

// The instantiation of the 128/64-row kernel for a launch: balanced or
// uniform unit plan, fp8 or bf16 K/V, head dim D.
template <int NW, int D = kHeadDim>
int launch_fwdh(bool bal, bool fp8, unsigned grid, hipStream_t hs,
                const FwdParams& fp) {
  const dim3 g(grid), b(NW * 64);
  if (fp8) {
    return bal ? launch(&attn_fwdh_kernel<NW, true, true, D>, g, b, hs, fp)
               : launch(&attn_fwdh_kernel<NW, false, true, D>, g, b, hs, fp);
  }
  return bal ? launch(&attn_fwdh_kernel<NW, true, false, D>, g, b, hs, fp)
             : launch(&attn_fwdh_kernel<NW, false, false, D>, g, b, hs, fp);
}

// The instantiation of the 256-row kernel for a launch.
template <int D = kHeadDim>
int launch_fwd256(bool bal, bool fp8, unsigned grid, hipStream_t hs,
                  const FwdParams& fp) {
  const dim3 g(grid), b(512);
  if (fp8) {
    return bal ? launch(&attn_fwd256_kernel<true, true, D>, g, b, hs, fp)
               : launch(&attn_fwd256_kernel<false, true, D>, g, b, hs, fp);
  }
  return bal ? launch(&attn_fwd256_kernel<true, false, D>, g, b, hs, fp)
             : launch(&attn_fwd256_kernel<false, false, D>, g, b, hs, fp);
}


// Phases of a verify call: the split-KV + tree pass, then the LSE merge.
enum { kPhaseAttend = 1, kPhaseMerge = 2 };

int run_verify(int phases, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* page_table, int32_t max_pages_per_seq,
                     int32_t num_pages, int32_t page_size,
                     const int32_t* prefix_lens, const int32_t* tree_offsets,
                     const uint64_t* masks, int32_t mask_words,
                     int32_t num_seqs, int32_t total_nodes,
                     int32_t max_prefix_len, int32_t max_nodes,
                     int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, float scale, int32_t num_splits,
                     void* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream,
                     bool fp8 = false, const float* k_scale = nullptr,
                     const float* v_scale = nullptr, bool allow_d64 = false) {
  // head dim 64 (tree_attn_verify_ex only): both phases in one call
  const bool d64 = allow_d64 && head_dim == 64 &&
                   phases == (kPhaseAttend | kPhaseMerge);
  int st = check_verify_sizes(num_seqs, total_nodes, num_q_heads,
                              num_kv_heads, d64 ? kHeadDim : head_dim,
                              max_prefix_len, max_nodes, num_splits,
                              mask_words, max_pages_per_seq, num_pages,
                              page_size, scale);
  if (st != TREE_ATTN_OK) return st;
  if (num_seqs == 0 || total_nodes == 0) return TREE_ATTN_OK;
  if (!q || !k_cache || !v_cache || !page_table || !prefix_lens ||
      !tree_offsets || !masks || !out || !lse) {
    return TREE_ATTN_ERR_NULL;
  }

  Plan pl;
  st = make_plan(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                 max_prefix_len, max_nodes, page_size, num_splits, cu_count(),
                 &pl, d64 ? 64 : kHeadDim, (d64 ? 64 : kHeadDim) * (fp8 ? 1 : 2));
  if (st != TREE_ATTN_OK) return st;
  if (pl.ws_bytes > 0) {
    if (!workspace) return TREE_ATTN_ERR_WORKSPACE;
    if (workspace_bytes < pl.ws_bytes) return TREE_ATTN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) {
      return TREE_ATTN_ERR_WORKSPACE;
    }
  }

  FwdParams fp;
  fp.q = static_cast<const __bf16*>(q);
  fp.k = static_cast<const __bf16*>(k_cache);
  fp.v = static_cast<const __bf16*>(v_cache);
  fp.page_table = page_table;
  fp.prefix_lens = prefix_lens;
  fp.tree_offsets = tree_offsets;
  fp.masks = masks;
  fp.out = static_cast<__bf16*>(out);
  fp.lse = lse;
  fp.part_o = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) +
                                          kCounterBytes);
  fp.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        pl.part_ml_off);
  fp.k_scale = fp8 ? k_scale : nullptr;
  fp.v_scale = fp8 ? v_scale : nullptr;
  // Both phases in one call with split partials: the attention kernel's
  // last split workgroup of each row block merges it (no merge launch).
  const bool fused = (phases & kPhaseAttend) && (phases & kPhaseMerge) &&
                     pl.splits > 1 && pl.blocks <= kMergeCounters;
  fp.counters = fused ? static_cast<unsigned*>(workspace) : nullptr;
  fp.max_pps = max_pages_per_seq;
  fp.num_pages = num_pages;
  fp.log2_page = ilog2(page_size);
  fp.W = mask_words;
  fp.max_tokens = (int)std::min<long long>((long long)max_pages_per_seq * page_size,
                                           1LL << 30);
  fp.S = num_seqs;
  fp.N = total_nodes;
  fp.Hq = num_q_heads;
  fp.Hkv = num_kv_heads;
  fp.G = num_q_heads / num_kv_heads;
  fp.per_xcd = (pl.units + 7) / 8;
  fp.plan = split_params(pl, prefix_lens, tree_offsets, num_seqs, total_nodes,
                         num_kv_heads, fp.G, fp.max_tokens, max_prefix_len,
                         max_nodes, num_splits);
  fp.scale_log2 = scale * kLog2e;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = 8u * (unsigned)fp.per_xcd;
  if (phases & kPhaseAttend) {
    // balanced plans run the instantiations that carry the device plan
    const bool bal = fp.plan.uniform_chunk == 0;
    if (d64) {
      if (pl.rows == kRowsPerWG8) {
        st = launch_fwd256<64>(bal, fp8, grid, hs, fp);
      } else if (pl.rows == kRowsPerWG128) {
        st = launch_fwdh<8, 64>(bal, fp8, grid, hs, fp);
      } else {
        st = launch_fwdh<4, 64>(bal, fp8, grid, hs, fp);
      }
    } else if (pl.rows == kRowsPerWG8) {
      st = launch_fwd256(bal, fp8, grid, hs, fp);
    } else if (pl.rows == kRowsPerWG128) {
      st = launch_fwdh<8>(bal, fp8, grid, hs, fp);
    } else {
      st = launch_fwdh<4>(bal, fp8, grid, hs, fp);
    }
    if (st != TREE_ATTN_OK) return st;
  }

  if ((phases & kPhaseMerge) && pl.splits > 1 && !fused) {
    MergeParams mp;
    mp.part_o = fp.part_o;
    mp.part_ml = fp.part_ml;
    mp.out = fp.out;
    mp.lse = lse;
    mp.Hq = num_q_heads;
    mp.G = fp.G;
    mp.plan = fp.plan;
    const long long mgrid =
        (long long)pl.units * (pl.rows / kMergeRowsPerWG);
    st = d64 ? launch(&attn_merge_kernel<64>, dim3((unsigned)mgrid),
                      dim3(kMergeWaves * 64), hs, mp)
             : launch(&attn_merge_kernel<>, dim3((unsigned)mgrid),
                      dim3(kMergeWaves * 64), hs, mp);
    if (st != TREE_ATTN_OK) return st;
  }
  return TREE_ATTN_OK;
}

// ---- device scratch of tree_attn_verify_noalloc
//
// A file-scope device array, one copy per GPU, holding what a workspace
// holds for tree_attn_verify: the arrival counters, then the split
// partials.  In host code its name stands for a host-side shadow, not a
// device address: the device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is handed to
// kernels.
constexpr size_t kScratchBytes = TREE_ATTN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > kCounterBytes, "scratch holds the counters");

__global__ void zero_words_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch; the first call on a
// device looks it up and clears its counter area on `stream` (a kernel,
// not a memset, so that a captured graph replays it correctly).  Every
// call that completes leaves the counters at zero again.
int device_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TREE_ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TREE_ATTN_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess ||
          q == nullptr) {
        return TREE_ATTN_ERR_HIP;
      }
      const int st = launch(&zero_words_kernel,
                            dim3((kMergeCounters + 255) / 256), dim3(256),
                            stream, static_cast<unsigned*>(q),
                            kMergeCounters);
      if (st != TREE_ATTN_OK) return st;
      g_scratch[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return TREE_ATTN_OK;
}

// Tree construction with MS register slots per lane (MS >= ceil((B+1)/64));
// kStrict is the one-candidate-per-step build.
static_assert(TREE_ATTN_MAX_NODES / 64 + 1 <= 17,
              "the largest tree needs at most 17 slots per lane");
template <bool kStrict>
int launch_tree(int ms, dim3 grid, dim3 block, hipStream_t hs,
                const TreeParams& tp) {
  if (ms <= 1) return launch(&build_tree_kernel<1, kStrict>, grid, block, hs, tp);
  if (ms <= 2) return launch(&build_tree_kernel<2, kStrict>, grid, block, hs, tp);
  if (ms <= 3) return launch(&build_tree_kernel<3, kStrict>, grid, block, hs, tp);
  if (ms <= 4) return launch(&build_tree_kernel<4, kStrict>, grid, block, hs, tp);
  if (ms <= 5) return launch(&build_tree_kernel<5, kStrict>, grid, block, hs, tp);
  if (ms <= 6) return launch(&build_tree_kernel<6, kStrict>, grid, block, hs, tp);
  if (ms <= 8) return launch(&build_tree_kernel<8, kStrict>, grid, block, hs, tp);
  if (ms <= 16) return launch(&build_tree_kernel<16, kStrict>, grid, block, hs, tp);
  return launch(&build_tree_kernel<17, kStrict>, grid, block, hs, tp);
}

}  // namespace

extern "C" {

const char* tree_attn_status_string(int status) {
  switch (status) {
    case TREE_ATTN_OK: return "ok";
    case TREE_ATTN_ERR_NULL: return "null pointer argument";
    case TREE_ATTN_ERR_SHAPE: return "inconsistent sizes";
    case TREE_ATTN_ERR_UNSUPPORTED: return "unsupported size";
    case TREE_ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case TREE_ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int tree_attn_abi_version(void) { return kAbiVersion; }

int tree_attn_build_mask(const int32_t* parents, const int32_t* tree_offsets,
                         int32_t num_seqs, int32_t total_nodes,
                         int32_t max_nodes, int32_t mask_words,
                         uint64_t* masks, int32_t* bad_node, void* stream) {
  if (num_seqs < 0 || total_nodes < 0 || max_nodes < 0 || mask_words < 1) {
    return TREE_ATTN_ERR_SHAPE;
  }
  if (mask_words > kMaskMaxWords || max_nodes > TREE_ATTN_MAX_NODES) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if ((long long)mask_words * 64 < max_nodes) return TREE_ATTN_ERR_SHAPE;
  if (num_seqs == 0) return TREE_ATTN_OK;
  if (!tree_offsets || !bad_node) return TREE_ATTN_ERR_NULL;
  if (total_nodes > 0 && (!parents || !masks)) return TREE_ATTN_ERR_NULL;

  const int cap = std::max(1, max_nodes);
  // one thread per node of the largest tree, whole waves
  const int threads = std::min(kMaskThreads, (cap + 63) / 64 * 64);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return launch(&build_mask_kernel, dim3(num_seqs), dim3(threads), st, parents,
                tree_offsets, num_seqs, total_nodes, cap, (int)mask_words,
                masks, bad_node);
}

void plan_info(const Plan& pl, int32_t* info) {
  info[0] = pl.rows == kRowsPerWG64 ? 4 : kWaves;
  info[1] = pl.rows;
  info[2] = pl.splits;
  info[3] = pl.chunk;
  info[4] = 8 * ((pl.units + 7) / 8);
}

// Cache formats of tree_attn_verify_ex: bf16 or FP8 E4M3 K/V with head
// dim 64 or 128, all on the tuned kernels.
bool ex_format_ok(int32_t kv_dtype, int32_t head_dim) {
  return (kv_dtype == TREE_ATTN_KV_BF16 ||
          kv_dtype == TREE_ATTN_KV_FP8_E4M3) &&
         (head_dim == 64 || head_dim == kHeadDim);
}

// Workspace of the tuned kernels' plan (the same for bf16 and fp8 K/V;
// head dim 64 only for tree_attn_verify_ex's calls).
size_t tuned_workspace_size(int32_t num_seqs, int32_t total_nodes,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_prefix_len,
                            int32_t max_nodes, int32_t page_size,
                            int32_t num_splits, bool allow_d64 = false,
                            bool fp8 = false) {
  const bool d64 = allow_d64 && head_dim == 64;
  if (check_sizes(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                  d64 ? kHeadDim : head_dim, max_prefix_len,
                  max_nodes) != TREE_ATTN_OK ||
      num_splits < 0 || !is_pow2(page_size) || page_size > 4096) {
    return 0;
  }
  if (num_seqs == 0 || total_nodes == 0) return 0;
  Plan pl;
  if (make_plan(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                max_prefix_len, max_nodes, page_size, num_splits, cu_count(),
                &pl, d64 ? 64 : kHeadDim,
                (d64 ? 64 : kHeadDim) * (fp8 ? 1 : 2)) != TREE_ATTN_OK) {
    return 0;
  }
  return pl.ws_bytes;
}

size_t tree_attn_workspace_size(int32_t num_seqs, int32_t total_nodes,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_prefix_len,
                                int32_t max_nodes, int32_t page_size,
                                int32_t num_splits) {
  return tuned_workspace_size(num_seqs, total_nodes, num_q_heads,
                              num_kv_heads, head_dim, max_prefix_len,
                              max_nodes, page_size, num_splits);
}

// The tuned kernels' launch for these sizes (bf16 or fp8 K/V; head dim 64
// only for tree_attn_verify_ex's calls: the plan does not depend on it).
int describe_tuned(int32_t num_seqs, int32_t total_nodes, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim,
                   int32_t max_prefix_len, int32_t max_nodes,
                   int32_t page_size, int32_t num_splits, int32_t* info,
                   bool allow_d64 = false, bool fp8 = false) {
  if (info == nullptr) return TREE_ATTN_ERR_NULL;
  const bool d64 = allow_d64 && head_dim == 64;
  int st = check_sizes(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                       d64 ? kHeadDim : head_dim, max_prefix_len, max_nodes);
  if (st != TREE_ATTN_OK) return st;
  if (num_splits < 0 || !is_pow2(page_size) || page_size > 4096) {
    return TREE_ATTN_ERR_SHAPE;
  }
  Plan pl;
  st = make_plan(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                 max_prefix_len, max_nodes, page_size, num_splits, cu_count(),
                 &pl, d64 ? 64 : kHeadDim, (d64 ? 64 : kHeadDim) * (fp8 ? 1 : 2));
  if (st != TREE_ATTN_OK) return st;
  plan_info(pl, info);
  return TREE_ATTN_OK;
}

int tree_attn_describe_plan(int32_t num_seqs, int32_t total_nodes,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_prefix_len,
                            int32_t max_nodes, int32_t page_size,
                            int32_t num_splits, int32_t* info) {
  return describe_tuned(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                        head_dim, max_prefix_len, max_nodes, page_size,
                        num_splits, info);
}

int tree_attn_describe_plan_ex(int32_t kv_dtype, int32_t num_seqs,
                               int32_t total_nodes, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_prefix_len, int32_t max_nodes,
                               int32_t page_size, int32_t num_splits,
                               int32_t* info) {
  if (info == nullptr) return TREE_ATTN_ERR_NULL;
  if (!ex_format_ok(kv_dtype, head_dim)) return TREE_ATTN_ERR_UNSUPPORTED;
  return describe_tuned(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                        head_dim, max_prefix_len, max_nodes, page_size,
                        num_splits, info, true,
                        kv_dtype == TREE_ATTN_KV_FP8_E4M3);
}

int tree_attn_verify(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* page_table, int32_t max_pages_per_seq,
                     int32_t num_pages, int32_t page_size,
                     const int32_t* prefix_lens, const int32_t* tree_offsets,
                     const uint64_t* masks, int32_t mask_words,
                     int32_t num_seqs, int32_t total_nodes,
                     int32_t max_prefix_len, int32_t max_nodes,
                     int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, float scale, int32_t num_splits,
                     void* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return run_verify(kPhaseAttend | kPhaseMerge, q, k_cache, v_cache,
                    page_table, max_pages_per_seq, num_pages, page_size,
                    prefix_lens, tree_offsets, masks, mask_words, num_seqs,
                    total_nodes, max_prefix_len, max_nodes, num_q_heads,
                    num_kv_heads, head_dim, scale, num_splits, out, lse,
                    workspace, workspace_bytes, stream);
}

int tree_attn_verify_noalloc(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const uint64_t* masks, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t num_splits, void* out, float* lse,
    void* stream) {
  // the same checks as tree_attn_verify, and the scratch-size check, before
  // any HIP call
  int st = check_verify_sizes(num_seqs, total_nodes, num_q_heads,
                              num_kv_heads, head_dim, max_prefix_len,
                              max_nodes, num_splits, mask_words,
                              max_pages_per_seq, num_pages, page_size, scale);
  if (st != TREE_ATTN_OK) return st;
  if (num_seqs == 0 || total_nodes == 0) return TREE_ATTN_OK;
  Plan pl;
  st = make_plan(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                 max_prefix_len, max_nodes, page_size, num_splits, cu_count(),
                 &pl);
  if (st != TREE_ATTN_OK) return st;
  if (pl.ws_bytes > kScratchBytes) return TREE_ATTN_ERR_WORKSPACE;
  if (!q || !k_cache || !v_cache || !page_table || !prefix_lens ||
      !tree_offsets || !masks || !out || !lse) {
    return TREE_ATTN_ERR_NULL;
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = device_scratch(hs, &ws);
  if (st != TREE_ATTN_OK) return st;
  return run_verify(kPhaseAttend | kPhaseMerge, q, k_cache, v_cache,
                    page_table, max_pages_per_seq, num_pages, page_size,
                    prefix_lens, tree_offsets, masks, mask_words, num_seqs,
                    total_nodes, max_prefix_len, max_nodes, num_q_heads,
                    num_kv_heads, head_dim, scale, num_splits, out, lse, ws,
                    kScratchBytes, stream);
}

int tree_attn_verify_attend(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const uint64_t* masks, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t num_splits, void* out, float* lse,
    void* workspace, size_t workspace_bytes, void* stream) {
  return run_verify(kPhaseAttend, q, k_cache, v_cache, page_table,
                    max_pages_per_seq, num_pages, page_size, prefix_lens,
                    tree_offsets, masks, mask_words, num_seqs, total_nodes,
                    max_prefix_len, max_nodes, num_q_heads, num_kv_heads,
                    head_dim, scale, num_splits, out, lse, workspace,
                    workspace_bytes, stream);
}

int tree_attn_verify_merge(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const uint64_t* masks, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t num_splits, void* out, float* lse,
    void* workspace, size_t workspace_bytes, void* stream) {
  return run_verify(kPhaseMerge, q, k_cache, v_cache, page_table,
                    max_pages_per_seq, num_pages, page_size, prefix_lens,
                    tree_offsets, masks, mask_words, num_seqs, total_nodes,
                    max_prefix_len, max_nodes, num_q_heads, num_kv_heads,
                    head_dim, scale, num_splits, out, lse, workspace,
                    workspace_bytes, stream);
}

int tree_attn_build_tree(const float* logp, const int32_t* tokens,
                         int32_t num_seqs, int32_t depth, int32_t topk,
                         int32_t budget, int32_t width, int32_t* parents,
                         int32_t* node_tokens, int32_t* depths, float* scores,
                         int32_t* sizes, void* stream) {
  if (num_seqs < 0 || depth < 0 || topk < 1 || budget < 0 || width < 1) {
    return TREE_ATTN_ERR_SHAPE;
  }
  if (budget > TREE_ATTN_MAX_NODES || topk > kTreeMaxTopK ||
      (long long)depth * topk > kTreeMaxLogp) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0) return TREE_ATTN_OK;
  if (!sizes) return TREE_ATTN_ERR_NULL;
  if (depth > 0 && (!logp || !tokens)) return TREE_ATTN_ERR_NULL;
  if (budget > 0 && (!parents || !node_tokens || !depths || !scores)) {
    return TREE_ATTN_ERR_NULL;
  }
  TreeParams tp;
  tp.logp = logp;
  tp.tokens = tokens;
  tp.parents = parents;
  tp.out_tokens = node_tokens;
  tp.depths = depths;
  tp.scores = scores;
  tp.sizes = sizes;
  tp.D = depth;
  tp.K = topk;
  tp.B = budget;
  tp.W = width;
  // slots 0 .. budget, 64 per register of a lane
  const int ms = budget / 64 + 1;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(num_seqs), block(64);
  // (an instantiation per slot count up to 8: each extraction selects and
  // updates a lane's MS slots, so unused slots cost time)
  return width == 1 ? launch_tree<true>(ms, grid, block, hs, tp)
                    : launch_tree<false>(ms, grid, block, hs, tp);
}

int tree_attn_accept(const int32_t* parents, const int32_t* tree_offsets,
                     const uint64_t* masks, int32_t mask_words,
                     const int32_t* draft_tokens, const int32_t* target_tokens,
                     const int32_t* root_tokens, int32_t num_seqs,
                     int32_t total_nodes, int32_t max_nodes,
                     int32_t* accept_len, int32_t* accept_nodes,
                     int32_t* bonus_tokens, void* stream) {
  const int st = check_accept(parents, tree_offsets, masks, mask_words,
                              draft_tokens, target_tokens, root_tokens,
                              num_seqs, total_nodes, max_nodes, accept_len,
                              accept_nodes, bonus_tokens);
  if (st != TREE_ATTN_OK || num_seqs == 0) return st;
  // one thread per node of the largest tree, whole waves
  const int threads = (std::max(1, (int)max_nodes) + 63) / 64 * 64;
  const AcceptArgs ap = accept_args(parents, tree_offsets, masks, mask_words,
                                    draft_tokens, target_tokens, root_tokens,
                                    total_nodes, max_nodes, accept_len,
                                    accept_nodes, bonus_tokens);
  return launch(&accept_kernel, dim3(num_seqs), dim3(threads),
                reinterpret_cast<hipStream_t>(stream), ap);
}

int tree_attn_commit_kv(void* k_cache, void* v_cache,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        int32_t num_pages, int32_t page_size,
                        const int32_t* prefix_lens, const int32_t* accept_len,
                        const int32_t* accept_nodes, int32_t num_seqs,
                        int32_t max_nodes, int32_t token_bytes,
                        void* stream) {
  const int st = check_commit(k_cache, v_cache, page_table, max_pages_per_seq,
                              num_pages, page_size, prefix_lens, num_seqs,
                              max_nodes, token_bytes);
  if (st != TREE_ATTN_OK || num_seqs == 0 || max_nodes == 0) return st;
  if (!accept_len || !accept_nodes) return TREE_ATTN_ERR_NULL;
  const CommitParams cp = commit_params(
      k_cache, v_cache, page_table, max_pages_per_seq, num_pages, page_size,
      prefix_lens, accept_len, accept_nodes, max_nodes, token_bytes,
      kCommitThreads);
  const long long grid = (long long)num_seqs * cp.slices;
  if (grid > 0x7fffffffLL) return TREE_ATTN_ERR_UNSUPPORTED;
  return launch(&commit_kv_kernel, dim3((unsigned)grid), dim3(kCommitThreads),
                reinterpret_cast<hipStream_t>(stream), cp);
}

int tree_attn_accept_commit(
    const int32_t* parents, const int32_t* tree_offsets,
    const uint64_t* masks, int32_t mask_words, const int32_t* draft_tokens,
    const int32_t* target_tokens, const int32_t* root_tokens,
    int32_t num_seqs, int32_t total_nodes, int32_t max_nodes, void* k_cache,
    void* v_cache, const int32_t* page_table, int32_t max_pages_per_seq,
    int32_t num_pages, int32_t page_size, const int32_t* prefix_lens,
    int32_t token_bytes, int32_t* accept_len, int32_t* accept_nodes,
    int32_t* bonus_tokens, void* stream) {
  int st = check_accept(parents, tree_offsets, masks, mask_words,
                        draft_tokens, target_tokens, root_tokens, num_seqs,
                        total_nodes, max_nodes, accept_len, accept_nodes,
                        bonus_tokens);
  if (st != TREE_ATTN_OK) return st;
  st = check_commit(k_cache, v_cache, page_table, max_pages_per_seq,
                    num_pages, page_size, prefix_lens, num_seqs, max_nodes,
                    token_bytes);
  if (st != TREE_ATTN_OK || num_seqs == 0) return st;
  // one thread per node of the largest tree and per 16-byte column of the
  // slice, whole waves
  const int threads =
      std::max(kCommitThreads, (std::max(1, (int)max_nodes) + 63) / 64 * 64);
  const AcceptArgs ap = accept_args(parents, tree_offsets, masks, mask_words,
                                    draft_tokens, target_tokens, root_tokens,
                                    total_nodes, max_nodes, accept_len,
                                    accept_nodes, bonus_tokens);
  const CommitParams cp = commit_params(
      k_cache, v_cache, page_table, max_pages_per_seq, num_pages, page_size,
      prefix_lens, accept_len, accept_nodes, max_nodes, token_bytes, threads);
  const long long grid = (long long)num_seqs * cp.slices;
  if (grid > 0x7fffffffLL) return TREE_ATTN_ERR_UNSUPPORTED;
  return launch(&accept_commit_kernel, dim3((unsigned)grid), dim3(threads),
                reinterpret_cast<hipStream_t>(stream), ap, cp);
}

int tree_attn_gdn_verify(const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* state, const int32_t* tree_offsets,
                         const uint64_t* masks, int32_t mask_words,
                         int32_t num_seqs, int32_t total_nodes,
                         int32_t max_nodes, int32_t num_heads,
                         int32_t head_dim, void* out, float* u,
                         void* stream) {
  if (num_seqs < 0 || total_nodes < 0 || max_nodes < 0 || num_heads < 1 ||
      mask_words < 1) {
    return TREE_ATTN_ERR_SHAPE;
  }
  // one tree's rows of u must stay below 2^31 bytes (buffer ranges)
  if (head_dim != kHeadDim || max_nodes > kGdnMaxNodes ||
      num_heads > kGdnMaxHeads) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if ((long long)mask_words * 64 < max_nodes) return TREE_ATTN_ERR_SHAPE;
  if ((long long)num_seqs * num_heads > 0x7fffffffLL) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0 || total_nodes == 0) return TREE_ATTN_OK;
  if (!q || !k || !v || !g || !beta || !state || !tree_offsets || !masks ||
      !out || !u) {
    return TREE_ATTN_ERR_NULL;
  }
  GdnParams gp;
  gp.q = static_cast<const __bf16*>(q);
  gp.k = static_cast<const __bf16*>(k);
  gp.v = static_cast<const __bf16*>(v);
  gp.g = g;
  gp.beta = beta;
  gp.state = state;
  gp.tree_offsets = tree_offsets;
  gp.masks = masks;
  gp.out = static_cast<__bf16*>(out);
  gp.u = u;
  gp.H = num_heads;
  gp.W = mask_words;
  return launch(&gdn_verify_kernel, dim3((unsigned)(num_seqs * num_heads)),
                dim3(kGdnThreads), reinterpret_cast<hipStream_t>(stream), gp);
}

int tree_attn_gdn_commit(const void* k, const float* u, const float* g,
                         const int32_t* tree_offsets,
                         const int32_t* accept_len,
                         const int32_t* accept_nodes, int32_t num_seqs,
                         int32_t max_nodes, int32_t num_heads,
                         int32_t head_dim, float* state, void* stream) {
  if (num_seqs < 0 || max_nodes < 0 || num_heads < 1) {
    return TREE_ATTN_ERR_SHAPE;
  }
  if (head_dim != kHeadDim || max_nodes > TREE_ATTN_MAX_NODES) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if ((long long)num_seqs * num_heads > 0x7fffffffLL) {
    return TREE_ATTN_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0 || max_nodes == 0) return TREE_ATTN_OK;
  if (!k || !u || !g || !tree_offsets || !accept_len || !accept_nodes ||
      !state) {
    return TREE_ATTN_ERR_NULL;
  }
  GdnCommitParams cp;
  cp.k = static_cast<const __bf16*>(k);
  cp.u = u;
  cp.g = g;
  cp.tree_offsets = tree_offsets;
  cp.accept_len = accept_len;
  cp.accept_nodes = accept_nodes;
  cp.state = state;
  cp.H = num_heads;
  cp.max_nodes = max_nodes;
  return launch(&gdn_commit_kernel, dim3((unsigned)(num_seqs * num_heads)),
                dim3(kGdnThreads), reinterpret_cast<hipStream_t>(stream), cp);
}

size_t tree_attn_workspace_size_ex(int32_t kv_dtype, int32_t num_seqs,
                                   int32_t total_nodes, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_prefix_len, int32_t max_nodes,
                                   int32_t page_size, int32_t num_splits) {
  if (!ex_format_ok(kv_dtype, head_dim)) return 0;
  return tuned_workspace_size(num_seqs, total_nodes, num_q_heads,
                              num_kv_heads, head_dim, max_prefix_len,
                              max_nodes, page_size, num_splits, true,
                              kv_dtype == TREE_ATTN_KV_FP8_E4M3);
}

int tree_attn_verify_ex(const void* q, const void* k_cache,
                        const void* v_cache, int32_t kv_dtype,
                        const float* k_scale, const float* v_scale,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        int32_t num_pages, int32_t page_size,
                        const int32_t* prefix_lens,
                        const int32_t* tree_offsets, const uint64_t* masks,
                        int32_t mask_words, int32_t num_seqs,
                        int32_t total_nodes, int32_t max_prefix_len,
                        int32_t max_nodes, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, float scale,
                        int32_t num_splits, void* out, float* lse,
                        void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!ex_format_ok(kv_dtype, head_dim)) return TREE_ATTN_ERR_UNSUPPORTED;
  return run_verify(kPhaseAttend | kPhaseMerge, q, k_cache, v_cache,
                    page_table, max_pages_per_seq, num_pages, page_size,
                    prefix_lens, tree_offsets, masks, mask_words, num_seqs,
                    total_nodes, max_prefix_len, max_nodes, num_q_heads,
                    num_kv_heads, head_dim, scale, num_splits, out, lse,
                    workspace, workspace_bytes, stream,
                    kv_dtype == TREE_ATTN_KV_FP8_E4M3, k_scale, v_scale, true);
}

#ifdef TREE_ATTN_DEBUG
// Debug builds: the device values tree_attn_verify trusts, checked on host
// copies of them.  The kernels clamp what is out of range (a page id past
// the pool, a tree offset past N) so that no access leaves the buffers;
// this replays the planned launch's indexing on the host and names the
// first value that would have been clamped.
int tree_attn_debug_check_verify(
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const int32_t* parents, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_splits, int32_t* report) {
  if (!report) return TREE_ATTN_ERR_NULL;
  for (int i = 0; i < 4; ++i) report[i] = -1;
  report[0] = TREE_ATTN_DEBUG_OK;
  int st = check_verify_sizes(num_seqs, total_nodes, num_q_heads,
                              num_kv_heads, head_dim, max_prefix_len,
                              max_nodes, num_splits, mask_words,
                              max_pages_per_seq, num_pages, page_size, 1.f);
  if (st != TREE_ATTN_OK || num_seqs == 0 || total_nodes == 0) return st;
  if (!page_table || !prefix_lens || !tree_offsets || !parents) {
    return TREE_ATTN_ERR_NULL;
  }
  auto fail = [&](int kind, int s, long long idx, long long val) {
    report[0] = kind;
    report[1] = s;
    report[2] = (int32_t)idx;
    report[3] = (int32_t)val;
    return TREE_ATTN_ERR_SHAPE;
  };
  Plan pl;
  st = make_plan(num_seqs, total_nodes, num_q_heads, num_kv_heads,
                 max_prefix_len, max_nodes, page_size, num_splits, cu_count(),
                 &pl);
  if (st != TREE_ATTN_OK) return st;
  const int log2_page = ilog2(page_size);
  const long long max_tokens = (long long)max_pages_per_seq * page_size;
  if (tree_offsets[0] != 0) return fail(TREE_ATTN_DEBUG_OFFSETS, 0, 0,
                                        tree_offsets[0]);
  for (int s = 0; s < num_seqs; ++s) {
    const int a = tree_offsets[s], b = tree_offsets[s + 1];
    if (b < a || b > total_nodes) {
      return fail(TREE_ATTN_DEBUG_OFFSETS, s, s + 1, b);
    }
    if (b - a > max_nodes) return fail(TREE_ATTN_DEBUG_TREE_SIZE, s, 0, b - a);
    const int P = prefix_lens[s];
    if (P < 0 || P > max_prefix_len) {
      return fail(TREE_ATTN_DEBUG_PREFIX, s, 0, P);
    }
    for (int i = 0; i < b - a; ++i) {
      const int par = parents[a + i];
      if (par < -1 || par >= i) return fail(TREE_ATTN_DEBUG_PARENT, s, i, par);
    }
    const long long T = (long long)P + (b - a);
    if (T > max_tokens) return fail(TREE_ATTN_DEBUG_TABLE, s, 0, T);
    // the pages each split of the plan reads, through its LDS copy of the
    // split's slice of the page table
    for (long long kbeg = 0; kbeg < T; kbeg += pl.chunk) {
      const long long kend = std::min(T, kbeg + pl.chunk);
      const long long lp0 = kbeg >> log2_page;
      const long long lp1 = (kend - 1) >> log2_page;
      if (lp1 - lp0 + 1 > kPageCache) {
        return fail(TREE_ATTN_DEBUG_PAGE_CACHE, s, lp1, lp1 - lp0 + 1);
      }
      for (long long lp = lp0; lp <= lp1; ++lp) {
        const int pg = page_table[(size_t)s * max_pages_per_seq + lp];
        if (pg < 0 || pg >= num_pages) {
          return fail(TREE_ATTN_DEBUG_PAGE_ID, s, lp, pg);
        }
      }
    }
  }
  if (tree_offsets[num_seqs] != total_nodes) {
    return fail(TREE_ATTN_DEBUG_OFFSETS, num_seqs, num_seqs,
                tree_offsets[num_seqs]);
  }
  return TREE_ATTN_OK;
}
#endif  // TREE_ATTN_DEBUG

}  // extern "C"
