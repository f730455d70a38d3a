// Host side of libpkv: block pool, RoPE table, validation, status strings.
#include <cmath>
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
