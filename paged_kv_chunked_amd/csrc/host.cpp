// Host side of libpkv: block pool, radix-tree prefix cache, RoPE table,
// validation, status strings.
#include <array>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "pkv_internal.h"

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer";
    case PKV_ERR_SHAPE: return "unsupported or inconsistent shape";
    case PKV_ERR_DTYPE: return "unsupported dtype";
    case PKV_ERR_RANGE: return "value out of range";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_NOMEM: return "block pool exhausted";
    case PKV_ERR_REFCOUNT: return "reference count misuse";
    case PKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

// The build passes the hash of the sources and flags it compiled.
#ifndef PKV_SOURCE_HASH
#error "PKV_SOURCE_HASH must be defined by the build"
#endif
const char* pkv_source_hash(void) { return PKV_SOURCE_HASH; }

// ---------------------------------------------------------------------------
// RoPE table: Kshipra part 3, section 4 (RoPE at absolute positions).  fp64,
// (cos, sin) of pos * theta^(-2i/D) from the C library, [max_pos][D/2][2].
// ---------------------------------------------------------------------------
pkv_status pkv_rope_table_bytes(int32_t head_dim, int32_t max_pos, size_t* bytes) {
  if (!bytes) return PKV_ERR_NULL;
  if (head_dim < 2 || head_dim % 2 || head_dim > 256) return PKV_ERR_SHAPE;
  if (max_pos < 1) return PKV_ERR_RANGE;
  *bytes = (size_t)max_pos * (size_t)(head_dim / 2) * 2 * sizeof(double);
  return PKV_OK;
}

pkv_status pkv_rope_table_host(double* cs, double theta, int32_t head_dim, int32_t max_pos) {
  size_t bytes;
  pkv_status st = pkv_rope_table_bytes(head_dim, max_pos, &bytes);
  if (st != PKV_OK) return st;
  if (!cs) return PKV_ERR_NULL;
  if (!(theta > 0.0)) return PKV_ERR_RANGE;
  const int half = head_dim / 2;
  std::vector<double> inv(half);
  for (int i = 0; i < half; ++i) inv[i] = std::pow(theta, -(2.0 * i) / (double)head_dim);
  for (int p = 0; p < max_pos; ++p) {
    const double fp = (double)p;
    double* row = cs + (size_t)p * half * 2;
    for (int i = 0; i < half; ++i) {
      const double a = fp * inv[i];
      row[2 * i] = std::cos(a);
      row[2 * i + 1] = std::sin(a);
    }
  }
  return PKV_OK;
}

pkv_status pkv_rope_table_init(void* d_cs, double theta, int32_t head_dim, int32_t max_pos,
                               void* stream) {
  size_t bytes;
  pkv_status st = pkv_rope_table_bytes(head_dim, max_pos, &bytes);
  if (st != PKV_OK) return st;
  if (!d_cs) return PKV_ERR_NULL;
  std::vector<double> h;
  try {
    h.resize(bytes / sizeof(double));
  } catch (const std::bad_alloc&) {
    return PKV_ERR_RANGE;
  }
  st = pkv_rope_table_host(h.data(), theta, head_dim, max_pos);
  if (st != PKV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(d_cs, h.data(), bytes, hipMemcpyHostToDevice, s) != hipSuccess)
    return PKV_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// Block pool: Kshipra part 3, section 1 (LIFO free list) and section 3
// (reference counts, copy-on-write).
// ---------------------------------------------------------------------------
}  // extern "C"

struct pkv_pool {
  std::vector<int32_t> free_list;  // back() is the next block handed out
  std::vector<int32_t> rc;
};

extern "C" {

pkv_pool* pkv_pool_create(int32_t num_blocks) {
  if (num_blocks < 1) return nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return nullptr;
  try {
    p->free_list.resize(num_blocks);
    p->rc.assign(num_blocks, 0);
  } catch (const std::bad_alloc&) {
    delete p;
    return nullptr;
  }
  for (int32_t i = 0; i < num_blocks; ++i) p->free_list[i] = i;
  return p;
}

void pkv_pool_destroy(pkv_pool* p) { delete p; }

pkv_status pkv_pool_alloc(pkv_pool* p, int32_t* id) {
  if (!p || !id) return PKV_ERR_NULL;
  if (p->free_list.empty()) return PKV_ERR_NOMEM;
  *id = p->free_list.back();
  p->free_list.pop_back();
  p->rc[*id] = 1;
  return PKV_OK;
}

pkv_status pkv_pool_alloc_n(pkv_pool* p, int32_t n, int32_t* ids) {
  if (!p || (n > 0 && !ids)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_RANGE;
  if ((size_t)n > p->free_list.size()) return PKV_ERR_NOMEM;
  for (int32_t i = 0; i < n; ++i) pkv_pool_alloc(p, ids + i);
  return PKV_OK;
}

static bool in_range(const pkv_pool* p, int32_t id) {
  return id >= 0 && (size_t)id < p->rc.size();
}

pkv_status pkv_pool_incref(pkv_pool* p, int32_t id) {
  if (!p) return PKV_ERR_NULL;
  if (!in_range(p, id)) return PKV_ERR_RANGE;
  if (p->rc[id] < 1) return PKV_ERR_REFCOUNT;
  ++p->rc[id];
  return PKV_OK;
}

pkv_status pkv_pool_decref(pkv_pool* p, int32_t id) {
  if (!p) return PKV_ERR_NULL;
  if (!in_range(p, id)) return PKV_ERR_RANGE;
  if (p->rc[id] < 1) return PKV_ERR_REFCOUNT;
  if (--p->rc[id] == 0) p->free_list.push_back(id);
  return PKV_OK;
}

pkv_status pkv_pool_cow(pkv_pool* p, int32_t id, int32_t* out_id, int32_t* copied) {
  if (!p || !out_id || !copied) return PKV_ERR_NULL;
  if (!in_range(p, id)) return PKV_ERR_RANGE;
  if (p->rc[id] < 1) return PKV_ERR_REFCOUNT;
  if (p->rc[id] == 1) {
    *out_id = id;
    *copied = 0;
    return PKV_OK;
  }
  int32_t nb;
  pkv_status st = pkv_pool_alloc(p, &nb);  // pop first: the old block stays shared
  if (st != PKV_OK) return st;
  --p->rc[id];
  *out_id = nb;
  *copied = 1;
  return PKV_OK;
}

int32_t pkv_pool_num_free(const pkv_pool* p) { return p ? (int32_t)p->free_list.size() : -1; }

int32_t pkv_pool_can_admit(const pkv_pool* p, int64_t evictable, int64_t active_reserved,
                           int64_t new_need) {
  if (!p || evictable < 0 || active_reserved < 0 || new_need < 0) return -1;
  return (int64_t)p->free_list.size() + evictable >= active_reserved + new_need ? 1 : 0;
}

int32_t pkv_pool_refcount(const pkv_pool* p, int32_t id) {
  if (!p || !in_range(p, id)) return -1;
  return p->rc[id];
}

pkv_status pkv_pool_free_list(const pkv_pool* p, int32_t* out, int32_t cap, int32_t* n) {
  if (!p || !n) return PKV_ERR_NULL;
  const int32_t len = (int32_t)p->free_list.size();
  *n = len;
  if (cap > 0 && !out) return PKV_ERR_NULL;
  for (int32_t i = 0; i < len && i < cap; ++i) out[i] = p->free_list[i];
  return PKV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Radix-tree prefix cache (Kshipra part 3, section 3).  Node 0 is the root;
// every other live node is one full block of 16 token ids and holds one
// reference to its physical block in the pool.  Children are found by a
// linear scan of the parent's child list (fan-out is small: distinct
// continuations of one prefix).
namespace {
struct RadixNode {
  std::array<int32_t, PKV_BLOCK_SIZE> key;
  int32_t block = -1;
  int32_t parent = -1;
  uint64_t last = 0;    // clock of the last match / insert that touched it
  int64_t serial = -1;  // creation order (LRU tie-break)
  bool alive = false;
  std::vector<int32_t> children;
};
}  // namespace

struct pkv_radix {
  pkv_pool* pool = nullptr;
  std::vector<RadixNode> nodes;
  std::vector<int32_t> free_nodes;
  uint64_t clock = 0;
  int64_t serial = 0;
  int32_t live = 0;
};

namespace {
int32_t find_child(const pkv_radix* r, int32_t node, const int32_t* key) {
  for (int32_t c : r->nodes[node].children)
    if (std::memcmp(r->nodes[c].key.data(), key, sizeof(int32_t) * PKV_BLOCK_SIZE) == 0)
      return c;
  return -1;
}

bool only_tree_holds(const pkv_radix* r, int32_t node) {
  const int32_t b = r->nodes[node].block;
  return r->pool->rc[b] == 1;
}

void remove_node(pkv_radix* r, int32_t node) {
  RadixNode& n = r->nodes[node];
  std::vector<int32_t>& sib = r->nodes[n.parent].children;
  for (size_t i = 0; i < sib.size(); ++i)
    if (sib[i] == node) {
      sib.erase(sib.begin() + i);
      break;
    }
  n.alive = false;
  n.children.clear();
  r->free_nodes.push_back(node);
  --r->live;
}
}  // namespace

extern "C" {

pkv_radix* pkv_radix_create(pkv_pool* pool) {
  if (!pool) return nullptr;
  pkv_radix* r = new (std::nothrow) pkv_radix;
  if (!r) return nullptr;
  r->pool = pool;
  r->nodes.resize(1);
  r->nodes[0].alive = true;
  return r;
}

void pkv_radix_destroy(pkv_radix* r) {
  if (!r) return;
  for (size_t i = 1; i < r->nodes.size(); ++i)
    if (r->nodes[i].alive) pkv_pool_decref(r->pool, r->nodes[i].block);
  delete r;
}

int32_t pkv_radix_match(pkv_radix* r, const int32_t* tokens, int32_t n, int32_t* blocks,
                        int32_t cap) {
  if (!r || n < 0 || (n > 0 && !tokens) || cap < 0 || (cap > 0 && !blocks)) return -1;
  ++r->clock;
  int32_t node = 0, m = 0;
  for (int32_t i = 0; i + PKV_BLOCK_SIZE <= n; i += PKV_BLOCK_SIZE) {
    const int32_t c = find_child(r, node, tokens + i);
    if (c < 0) break;
    r->nodes[c].last = r->clock;
    if (m < cap) blocks[m] = r->nodes[c].block;
    ++m;
    node = c;
  }
  return m;
}

pkv_status pkv_radix_insert(pkv_radix* r, const int32_t* tokens, int32_t n,
                            const int32_t* blocks) {
  if (!r) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_RANGE;
  const int32_t nb = n / PKV_BLOCK_SIZE;
  if (nb > 0 && (!tokens || !blocks)) return PKV_ERR_NULL;
  // validate first: every block that would become a new node must be live
  {
    int32_t node = 0, i = 0;
    for (; i < nb; ++i) {
      const int32_t c = find_child(r, node, tokens + (size_t)i * PKV_BLOCK_SIZE);
      if (c < 0) break;
      node = c;
    }
    for (; i < nb; ++i) {
      const int32_t b = blocks[i];
      if (!in_range(r->pool, b)) return PKV_ERR_RANGE;
      if (r->pool->rc[b] < 1) return PKV_ERR_REFCOUNT;
    }
  }
  try {
    ++r->clock;
    int32_t node = 0;
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t* key = tokens + (size_t)i * PKV_BLOCK_SIZE;
      int32_t c = find_child(r, node, key);
      if (c < 0) {
        if (!r->free_nodes.empty()) {
          c = r->free_nodes.back();
          r->free_nodes.pop_back();
        } else {
          c = (int32_t)r->nodes.size();
          r->nodes.emplace_back();
        }
        RadixNode& nn = r->nodes[c];
        std::memcpy(nn.key.data(), key, sizeof(int32_t) * PKV_BLOCK_SIZE);
        nn.block = blocks[i];
        nn.parent = node;
        nn.serial = r->serial++;
        nn.alive = true;
        r->nodes[node].children.push_back(c);
        ++r->live;
        pkv_pool_incref(r->pool, blocks[i]);
      }
      r->nodes[c].last = r->clock;
      node = c;
    }
  } catch (const std::bad_alloc&) {
    return PKV_ERR_NOMEM;
  }
  return PKV_OK;
}

int32_t pkv_radix_evict(pkv_radix* r, int32_t target) {
  if (!r || target < 0) return -1;
  int32_t freed = 0;
  while (freed < target) {
    // re-scan for the least recently used evictable leaf every iteration
    int32_t best = -1;
    for (size_t i = 1; i < r->nodes.size(); ++i) {
      const RadixNode& n = r->nodes[i];
      if (!n.alive || !n.children.empty() || !only_tree_holds(r, (int32_t)i)) continue;
      if (best < 0 || n.last < r->nodes[best].last ||
          (n.last == r->nodes[best].last && n.serial < r->nodes[best].serial))
        best = (int32_t)i;
    }
    if (best < 0) break;  // nothing evictable left
    const int32_t b = r->nodes[best].block;
    remove_node(r, best);
    pkv_pool_decref(r->pool, b);
    ++freed;
  }
  return freed;
}

int32_t pkv_radix_evictable(const pkv_radix* r) {
  if (!r) return -1;
  // post-order over the tree: a node counts if the tree alone holds its block
  // and its whole subtree counts
  std::vector<int32_t> order;
  std::vector<int32_t> stack{0};
  while (!stack.empty()) {
    const int32_t n = stack.back();
    stack.pop_back();
    order.push_back(n);
    for (int32_t c : r->nodes[n].children) stack.push_back(c);
  }
  std::vector<char> whole(r->nodes.size(), 1);
  int32_t count = 0;
  for (size_t k = order.size(); k-- > 1;) {  // children before parents; skip the root
    const int32_t n = order[k];
    bool ok = only_tree_holds(r, n);
    for (int32_t c : r->nodes[n].children) ok = ok && whole[c];
    whole[n] = ok;
    count += ok;
  }
  return count;
}

int32_t pkv_radix_num_nodes(const pkv_radix* r) { return r ? r->live : -1; }

// ---------------------------------------------------------------------------
pkv_status pkv_validate_tables(const pkv_geom* g, const int32_t* bt, int32_t max_blocks,
                               const int32_t* lens, int32_t num_seqs) {
  if (!g || (num_seqs > 0 && (!bt || !lens))) return PKV_ERR_NULL;
  if (max_blocks < 1 || num_seqs < 0) return PKV_ERR_SHAPE;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t L = lens[b];
    if (L < 0) return PKV_ERR_RANGE;
    const int64_t nb = ((int64_t)L + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
    if (nb > max_blocks) return PKV_ERR_RANGE;
    for (int64_t i = 0; i < nb; ++i) {
      const int32_t id = bt[(int64_t)b * max_blocks + i];
      if (id < 0 || id >= g->num_blocks) return PKV_ERR_RANGE;
    }
  }
  return PKV_OK;
}

pkv_status pkv_f64_to_f16_host(const double* x, uint16_t* out, int64_t n) {
  if (n > 0 && (!x || !out)) return PKV_ERR_NULL;
  for (int64_t i = 0; i < n; ++i) out[i] = pkv::f64_to_f16_bits(x[i]);
  return PKV_OK;
}

}  // extern "C"
