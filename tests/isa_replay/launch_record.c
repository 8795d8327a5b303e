/* A stand-in for the HIP runtime calls that the library's host code makes, for
 * replaying its kernels on the CPU.  Linked against a host-only build of the
 * library, it records every kernel launch -- kernel handle and name, grid,
 * block, dynamic LDS bytes and the bytes of each argument -- instead of running
 * it.  A name comes from the kernel's registration when the build registers
 * kernels, else from the loader for kernels of external linkage; the caller
 * resolves the rest from the handle.  Nothing here touches a GPU. */
#define _GNU_SOURCE
#include <dlfcn.h>
#include <stdint.h>
#include <string.h>

typedef struct {
  uint32_t x, y, z;
} dim3;

enum { MAX_LAUNCHES = 256, MAX_ARGS = 32, STRUCT_BYTES = 2048, MAX_KERNELS = 4096 };

typedef struct {
  char name[512];
  dim3 grid, block;
  size_t shmem;
  unsigned char arg0[STRUCT_BYTES]; /* the first argument (a kernel's parameter block) */
  unsigned char argv[MAX_ARGS][8];  /* the first 8 bytes of every argument */
  int nargs;
  const void* handle;               /* the kernel's host-side handle */
} launch_t;

static launch_t launches[MAX_LAUNCHES];
static int n_launches = 0;
static dim3 cfg_grid, cfg_block;
static size_t cfg_shmem;
static void* cfg_stream;

static const void* kernel_handle[MAX_KERNELS];
static char kernel_name[MAX_KERNELS][512];
static int n_kernels = 0;

/* argument counts of kernels that take more than one argument, set by the caller */
static char multi_name[256][512];
static int multi_count[256];
static int n_multi = 0;

void record_set_nargs(const char* name, int n) {
  if (n_multi < 256) {
    strncpy(multi_name[n_multi], name, 511);
    multi_count[n_multi++] = n;
  }
}

int record_count(void) { return n_launches; }
void record_clear(void) { n_launches = 0; }
const launch_t* record_get(int i) { return (i >= 0 && i < n_launches) ? &launches[i] : 0; }
int record_struct_size(void) { return (int)sizeof(launch_t); }

int __hipPushCallConfiguration(dim3 g, dim3 b, size_t s, void* st) {
  cfg_grid = g;
  cfg_block = b;
  cfg_shmem = s;
  cfg_stream = st;
  return 0;
}

int __hipPopCallConfiguration(dim3* g, dim3* b, size_t* s, void** st) {
  *g = cfg_grid;
  *b = cfg_block;
  *s = cfg_shmem;
  *st = cfg_stream;
  return 0;
}

int hipLaunchKernel(const void* f, dim3 g, dim3 b, void** args, size_t shm, void* st) {
  (void)st;
  if (n_launches >= MAX_LAUNCHES) return 1;
  launch_t* l = &launches[n_launches++];
  memset(l, 0, sizeof(*l));
  for (int i = 0; i < n_kernels; ++i)
    if (kernel_handle[i] == f) {
      strncpy(l->name, kernel_name[i], 511);
      break;
    }
  Dl_info di;
  if (!l->name[0] && dladdr(f, &di) && di.dli_sname) strncpy(l->name, di.dli_sname, 511);
  l->grid = g;
  l->block = b;
  l->shmem = shm;
  l->handle = f;
  l->nargs = 1;
  for (int i = 0; i < n_multi; ++i)
    if (strcmp(multi_name[i], l->name) == 0) l->nargs = multi_count[i];
  memcpy(l->arg0, args[0], STRUCT_BYTES);
  for (int i = 0; i < l->nargs && i < MAX_ARGS; ++i) memcpy(l->argv[i], args[i], 8);
  return 0;
}

int hipGetLastError(void) { return 0; }

int hipGetDevice(int* d) {
  *d = 0;
  return 0;
}

/* device-side static arrays resolve to a host buffer of the same role */
static unsigned char symbol_memory[64 << 20] __attribute__((aligned(256)));
void* record_symbol_memory(void) { return symbol_memory; }
size_t record_symbol_bytes(void) { return sizeof(symbol_memory); }

int hipGetSymbolAddress(void** p, const void* sym) {
  (void)sym;
  *p = symbol_memory;
  return 0;
}

void** __hipRegisterFatBinary(const void* data) {
  (void)data;
  static void* handle;
  return &handle;
}

void __hipUnregisterFatBinary(void** h) { (void)h; }

void __hipRegisterFunction(void** module, const void* host_fn, char* dev_fn, const char* dev_name,
                           int limit, void* tid, void* bid, void* bdim, void* gdim, int* wsize) {
  (void)module; (void)dev_fn; (void)limit; (void)tid; (void)bid; (void)bdim; (void)gdim; (void)wsize;
  if (n_kernels < MAX_KERNELS) {
    kernel_handle[n_kernels] = host_fn;
    strncpy(kernel_name[n_kernels++], dev_name, 511);
  }
}

void __hipRegisterVar(void** module, char* host_var, char* dev_var, const char* dev_name, int ext,
                      size_t size, int constant, int global) {
  (void)module; (void)host_var; (void)dev_var; (void)dev_name; (void)ext; (void)size; (void)constant;
  (void)global;
}
