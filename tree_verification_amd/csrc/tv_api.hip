// Shared host-side pieces of libtreeverify: device queries and status names.

#include "tv_common.h"

#include <dlfcn.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

namespace {
constexpr int kMaxDevices = 64;
int g_cu[kMaxDevices];
std::once_flag g_once[kMaxDevices];
}  // namespace

int tv_device_cu_count(int* cu_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TV_ERR_HIP;
  std::call_once(g_once[dev], [dev]() {
    hipDeviceProp_t prop;
    g_cu[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess) ? prop.multiProcessorCount : 0;
  });
  if (g_cu[dev] <= 0) return TV_ERR_HIP;
  *cu_out = g_cu[dev];
  return TV_OK;
}

namespace {

typedef int (*RangePushFn)(const char*);
typedef int (*RangePopFn)();
RangePushFn g_push = nullptr;
RangePopFn g_pop = nullptr;
bool g_trace = false, g_debug = false;
bool g_spin_set = false;
long long g_spin = 0;
std::once_flag g_env_once;

void read_env() {
  std::call_once(g_env_once, []() {
    const char* tr = getenv("TV_TRACE");
    const char* db = getenv("TV_DEBUG");
    const char* sp = getenv("TV_CHASE_SPIN_LIMIT");
    g_debug = db && *db && *db != '0';
    if (sp && *sp) {
      g_spin_set = true;
      g_spin = atoll(sp);
    }
    if (tr && *tr && *tr != '0') {
      for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so", "libroctx64.so"}) {
        void* h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
        if (!h) continue;
        g_push = (RangePushFn)dlsym(h, "roctxRangePushA");
        g_pop = (RangePopFn)dlsym(h, "roctxRangePop");
        if (g_push && g_pop) break;
        g_push = nullptr;
        g_pop = nullptr;
      }
      g_trace = g_push != nullptr;
    }
  });
}

template <typename T>
bool fetch(std::vector<T>& dst, const T* src, size_t n, hipStream_t stream) {
  dst.assign(n, T());
  if (n == 0) return true;
  if (hipStreamSynchronize(stream) != hipSuccess) return false;
  return hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

}  // namespace

TvTraceScope::TvTraceScope(const char* name) {
  read_env();
  on = g_trace;
  if (on) g_push(name);
}

TvTraceScope::~TvTraceScope() {
  if (on) g_pop();
}

bool tv_debug_enabled() {
  read_env();
  return g_debug;
}

long long tv_chase_spin_limit(long long dflt) {
  read_env();
  return g_spin_set ? g_spin : dflt;
}

int tv_debug_trees(const char* entry, const int32_t* parent, const int32_t* n_nodes, int batch, int n_max,
                   hipStream_t stream) {
  if (!tv_debug_enabled() || batch <= 0 || !parent || !n_nodes) return 0;
  std::vector<int32_t> par, nn;
  if (!fetch(par, parent, (size_t)batch * n_max, stream) || !fetch(nn, n_nodes, (size_t)batch, stream)) {
    fprintf(stderr, "[tv debug] %s: could not read the tree arrays\n", entry);
    return 0;
  }
  int bad = 0;
  for (int b = 0; b < batch; ++b) {
    const int n = nn[b];
    if (n < 1 || n > n_max) {
      fprintf(stderr, "[tv debug] %s: request %d: n_nodes %d outside [1, %d]\n", entry, b, n, n_max);
      ++bad;
      continue;
    }
    const int32_t* pr = par.data() + (size_t)b * n_max;
    for (int i = 0; i < n; ++i) {
      const bool ok = i == 0 ? pr[0] == -1 : (pr[i] >= 0 && pr[i] < i);
      if (!ok) {
        fprintf(stderr, "[tv debug] %s: request %d: parent[%d] = %d (need %s)\n", entry, b, i, pr[i],
                i == 0 ? "-1" : "0 <= parent[i] < i");
        ++bad;
        break;
      }
    }
  }
  return bad;
}

int tv_debug_kv(const char* entry, const int32_t* block_table, const int32_t* prefix_len, const int32_t* n_nodes,
                int batch, int max_blocks, int block_size, int num_blocks, hipStream_t stream) {
  if (!tv_debug_enabled() || batch <= 0 || !block_table || !prefix_len || !n_nodes) return 0;
  std::vector<int32_t> tab, pre, nn;
  if (!fetch(tab, block_table, (size_t)batch * max_blocks, stream) || !fetch(pre, prefix_len, (size_t)batch, stream) ||
      !fetch(nn, n_nodes, (size_t)batch, stream)) {
    fprintf(stderr, "[tv debug] %s: could not read the KV metadata\n", entry);
    return 0;
  }
  int bad = 0;
  for (int b = 0; b < batch; ++b) {
    const long long len = (long long)pre[b] + nn[b];
    if (pre[b] < 0 || len > (long long)max_blocks * block_size) {
      fprintf(stderr, "[tv debug] %s: request %d: prefix %d + %d nodes do not fit %d blocks of %d\n", entry, b,
              pre[b], nn[b], max_blocks, block_size);
      ++bad;
      continue;
    }
    const long long nblk = (len + block_size - 1) / block_size;
    for (long long i = 0; i < nblk; ++i) {
      const int id = tab[(size_t)b * max_blocks + i];
      if (id < 0 || id >= num_blocks) {
        fprintf(stderr, "[tv debug] %s: request %d: block_table[%lld] = %d outside the pool of %d\n", entry, b, i,
                id, num_blocks);
        ++bad;
        break;
      }
    }
  }
  return bad;
}

int tv_debug_finish(const char* entry, int rc, hipStream_t stream) {
  if (!tv_debug_enabled() || rc != TV_OK) return rc;
  const hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    fprintf(stderr, "[tv debug] %s: %s\n", entry, hipGetErrorString(e));
    return TV_ERR_HIP;
  }
  return rc;
}

extern "C" const char* tv_status_string(int code) {
  switch (code) {
    case TV_OK: return "TV_OK";
    case TV_ERR_INVALID_ARG: return "TV_ERR_INVALID_ARG";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED";
    case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE";
    case TV_ERR_HIP: return "TV_ERR_HIP";
    default: return "unknown status";
  }
}
