// Bundle order of a draft tree (host code): depth-first preorder from the root, the children of a
// node in increasing index.  Leaves under one branching node become adjacent, so verification rows
// that follow each other share their prefix (DiffSpec README, CGCL-codes, "Features": the bundle
// scheduler groups draft-tree leaves by branching ancestor for prefix-coherent verification), and
// every subtree becomes one index range, which turns the attention's ancestor test into two
// comparisons.
//
// O(n) with fixed-size stack arrays (no allocation):
//   1. child counts, then children grouped by parent in increasing index (a counting sort; the
//      nodes are visited in index order, so each group stays sorted);
//   2. subtree sizes, children before parents (indices decreasing, since parents[i] < i);
//   3. positions, parents before children: a node's first child sits right after it, each further
//      child after the previous child's whole subtree.
#include <cstdio>

#include "spec_internal.h"

namespace spec {
int host_fail(int status, const char* what);
}

extern "C" int spec_tree_bundle_order(const int32_t* parents, int32_t num_nodes, int32_t* order,
                                      int32_t* new_parents, int32_t* subtree_end, int32_t* bundle) {
  using spec::host_fail;
  constexpr int kMax = spec::kMaxTreeNodes;
  if (num_nodes < 0) return host_fail(SPEC_ERR_INVALID_ARGUMENT, "num_nodes: must be >= 0");
  if (num_nodes > kMax) return host_fail(SPEC_ERR_UNSUPPORTED, "num_nodes: supported up to SPEC_MAX_TREE_NODES");
  if (num_nodes == 0) return host_fail(SPEC_OK, nullptr);
  if (!parents) return host_fail(SPEC_ERR_INVALID_ARGUMENT, "parents: NULL");
  if (!order) return host_fail(SPEC_ERR_INVALID_ARGUMENT, "order: NULL");
  if (!subtree_end) return host_fail(SPEC_ERR_INVALID_ARGUMENT, "subtree_end: NULL");
  if (parents[0] != -1) return host_fail(SPEC_ERR_INVALID_ARGUMENT, "parents[0]: must be -1 (the root)");
  for (int32_t i = 1; i < num_nodes; ++i) {
    if (parents[i] < 0 || parents[i] >= i) {
      char buf[96];
      snprintf(buf, sizeof(buf), "parents[%d] = %d: must satisfy 0 <= parent < %d", i, parents[i], i);
      return host_fail(SPEC_ERR_INVALID_ARGUMENT, buf);
    }
  }
  const int n = num_nodes;
  int first[kMax + 1];       // children of u: kids[first[u] .. first[u + 1])
  int kids[kMax];
  int size[kMax], pos[kMax], branch[kMax];
  for (int u = 0; u <= n; ++u) first[u] = 0;
  for (int i = 1; i < n; ++i) ++first[parents[i] + 1];
  for (int u = 0; u < n; ++u) first[u + 1] += first[u];
  {
    int fill[kMax];
    for (int u = 0; u < n; ++u) fill[u] = first[u];
    for (int i = 1; i < n; ++i) kids[fill[parents[i]]++] = i;
  }
  for (int u = 0; u < n; ++u) size[u] = 1;
  for (int i = n - 1; i > 0; --i) size[parents[i]] += size[i];
  pos[0] = 0;
  branch[0] = 0;             // the root's bundle is the root
  for (int u = 0; u < n; ++u) {
    int next = pos[u] + 1;
    const bool branching = first[u + 1] - first[u] >= 2;
    for (int k = first[u]; k < first[u + 1]; ++k) {
      const int c = kids[k];
      pos[c] = next;
      next += size[c];
      branch[c] = branching ? u : branch[u];
    }
  }
  for (int u = 0; u < n; ++u) {
    const int i = pos[u];
    order[i] = u;
    subtree_end[i] = i + size[u];
    if (new_parents) new_parents[i] = u == 0 ? -1 : pos[parents[u]];
    if (bundle) bundle[i] = pos[branch[u]];
  }
  return host_fail(SPEC_OK, nullptr);
}
