// Host-side checks of the C ABI under AddressSanitizer, with the debug
// checker of a TREE_ATTN_DEBUG build (no GPU needed: every call here fails
// or finishes in its host-side checks, or reads host arrays only).
// Built and run by tests/test_debug_build.py; prints one line per failed
// expectation and exits with the number of failures.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tree_attn.h"
#include "tree_attn_debug.h"

static int g_fail = 0;

#define EXPECT_EQ(got, want)                                              \
  do {                                                                    \
    const long long g_ = (long long)(got), w_ = (long long)(want);        \
    if (g_ != w_) {                                                       \
      std::printf("FAIL line %d: %s = %lld, expected %lld\n", __LINE__,   \
                  #got, g_, w_);                                          \
      ++g_fail;                                                           \
    }                                                                     \
  } while (0)

// a non-null stand-in for device pointers: the calls below return before
// any of them is dereferenced or passed to HIP
static void* const kDev = reinterpret_cast<void*>(0x1000);

static int verify_call(int S, int N, int Hq, int Hkv, int d, int W,
                       int max_p, int max_b, int page, int splits,
                       size_t ws_bytes, bool null_q = false) {
  return tree_attn_verify(null_q ? nullptr : kDev, kDev, kDev,
                          (const int32_t*)kDev, 64, 64, page,
                          (const int32_t*)kDev, (const int32_t*)kDev,
                          (const uint64_t*)kDev, W, S, N, max_p, max_b, Hq,
                          Hkv, d, 0.088f, splits, kDev, (float*)kDev,
                          ws_bytes ? kDev : nullptr, ws_bytes, nullptr);
}

struct Inputs {
  int S, N, max_p, max_b, pps, num_pages, page;
  std::vector<int32_t> table, prefix, offs, parents;
};

// S sequences of prefix P and tree B, pages numbered in order
static Inputs make_inputs(int S, int P, int B, int page) {
  Inputs in;
  in.S = S;
  in.N = S * B;
  in.max_p = P;
  in.max_b = B;
  in.page = page;
  in.pps = (P + B + page - 1) / page;
  in.num_pages = S * in.pps;
  for (int s = 0; s < S; ++s) {
    for (int i = 0; i < in.pps; ++i) in.table.push_back(s * in.pps + i);
    in.prefix.push_back(P);
    in.offs.push_back(s * B);
    for (int i = 0; i < B; ++i) in.parents.push_back(i - 1);
  }
  in.offs.push_back(S * B);
  return in;
}

static int check(const Inputs& in, int32_t* rep, int splits = 0) {
  return tree_attn_debug_check_verify(
      in.table.data(), in.pps, in.num_pages, in.page, in.prefix.data(),
      in.offs.data(), in.parents.data(), (in.max_b + 63) / 64, in.S, in.N,
      in.max_p, in.max_b, 32, 8, 128, splits, rep);
}

int main() {
  // ---- argument checks of the launch entry points (before any HIP call)
  EXPECT_EQ(verify_call(1, 16, 8, 3, 128, 1, 256, 16, 16, 0, 0),
            TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(verify_call(1, 16, 8, 2, 64, 1, 256, 16, 16, 0, 0),
            TREE_ATTN_ERR_UNSUPPORTED);
  EXPECT_EQ(verify_call(1, 16, 8, 2, 128, 1, 256, 65, 16, 0, 0),
            TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(verify_call(1, 16, 8, 2, 128, 1, 256, 16, 12, 0, 0),
            TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(verify_call(1, 16, 8, 2, 128, 1, 256, 16, 16, 0, 0, true),
            TREE_ATTN_ERR_NULL);
  EXPECT_EQ(verify_call(1, 16, 8, 2, 128, 1, 256, 16, 16, 4, 0),
            TREE_ATTN_ERR_WORKSPACE);
  EXPECT_EQ(verify_call(0, 0, 8, 2, 128, 1, 256, 16, 16, 0, 0), TREE_ATTN_OK);
  int32_t bad[1];
  EXPECT_EQ(tree_attn_build_mask(nullptr, nullptr, 1, 4, 4, 1, nullptr, bad,
                                 nullptr),
            TREE_ATTN_ERR_NULL);
  EXPECT_EQ(tree_attn_build_mask((const int32_t*)kDev, (const int32_t*)kDev,
                                 1, 200, 200, 2, (uint64_t*)kDev, bad,
                                 nullptr),
            TREE_ATTN_ERR_SHAPE);
  int32_t info[5];
  EXPECT_EQ(tree_attn_describe_plan(1, 16, 8, 2, 128, 256, 16, 16, 0,
                                    nullptr),
            TREE_ATTN_ERR_NULL);

  // ---- planning over a sweep of shapes: every plan is internally
  // consistent and every forced split needs a workspace
  const int heads[][2] = {{8, 2}, {32, 8}, {32, 4}, {4, 4}, {2, 1}};
  for (auto& h : heads) {
    for (int P : {0, 1, 255, 4096, 32768, 200000}) {
      for (int B : {1, 16, 64, 256, 1024}) {
        for (int page : {1, 16, 64}) {
          for (int splits : {0, 1, 3, 64}) {
            const int st = tree_attn_describe_plan(4, 4 * B, h[0], h[1], 128,
                                                   P, B, page, splits, info);
            if (st != TREE_ATTN_OK) {
              EXPECT_EQ(st, TREE_ATTN_ERR_UNSUPPORTED);
              continue;
            }
            const long long T = (long long)P + B;
            // 64-row blocks run four waves, 128- and 256-row blocks eight
            EXPECT_EQ(info[0], info[1] == 64 ? 4 : 8);
            EXPECT_EQ(info[1] == 64 || info[1] == 128 || info[1] == 256, 1);
            const int G = h[0] / h[1];
            EXPECT_EQ(info[1] != 64 || G * B <= 128, 1);
            EXPECT_EQ(info[3] % 64, 0);
            EXPECT_EQ((long long)info[2] * info[3] >= T, 1);
            EXPECT_EQ((long long)(info[2] - 1) * info[3] < T, 1);
            EXPECT_EQ(info[3] <= 1039LL * page || info[3] == 64, 1);
            const size_t ws = tree_attn_workspace_size(
                4, 4 * B, h[0], h[1], 128, P, B, page, splits);
            EXPECT_EQ(ws > 0, info[2] > 1);
          }
        }
      }
    }
  }

  // ---- the debug checker on host arrays
  int32_t rep[4];
  Inputs ok = make_inputs(3, 100, 20, 16);
  EXPECT_EQ(check(ok, rep), TREE_ATTN_OK);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_OK);
  EXPECT_EQ(check(ok, rep, 5), TREE_ATTN_OK);

  Inputs pg = ok;
  pg.table[1 * pg.pps + 3] = pg.num_pages;  // past the pool
  EXPECT_EQ(check(pg, rep), TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_PAGE_ID);
  EXPECT_EQ(rep[1], 1);
  EXPECT_EQ(rep[2], 3);
  EXPECT_EQ(rep[3], pg.num_pages);
  pg.table[1 * pg.pps + 3] = -2;
  EXPECT_EQ(check(pg, rep, 3), TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_PAGE_ID);

  Inputs pre = ok;
  pre.prefix[2] = pre.max_p + 1;
  EXPECT_EQ(check(pre, rep), TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_PREFIX);
  EXPECT_EQ(rep[1], 2);

  Inputs par = ok;
  par.parents[20 + 7] = 7;  // parent[i] = i
  EXPECT_EQ(check(par, rep), TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_PARENT);
  EXPECT_EQ(rep[1], 1);
  EXPECT_EQ(rep[2], 7);

  Inputs off = ok;
  off.offs[2] = off.offs[1] - 1;
  EXPECT_EQ(check(off, rep), TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_OFFSETS);

  Inputs big = ok;
  big.offs[1] = 30;  // a tree of 30 nodes > max_nodes 20
  big.offs[2] = 40;
  EXPECT_EQ(check(big, rep), TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_TREE_SIZE);

  Inputs tab = make_inputs(1, 100, 20, 16);
  tab.pps -= 1;  // the table covers one page less than the tokens
  EXPECT_EQ(check(tab, rep), TREE_ATTN_ERR_SHAPE);
  EXPECT_EQ(rep[0], TREE_ATTN_DEBUG_TABLE);

  EXPECT_EQ(check(ok, nullptr), TREE_ATTN_ERR_NULL);

  std::printf("%s: %d failure(s)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail;
}
