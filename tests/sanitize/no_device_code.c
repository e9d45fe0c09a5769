/*
 * Registration hooks for a host-only build of the library (the .hip files
 * compiled with --cuda-host-only: kernel launchers without device code).
 * Every object's static constructor registers its (absent) code object and
 * kernels; these no-op definitions take the place of the HIP runtime's, so
 * the executable starts without a code object.  No kernel is ever launched
 * by the host driver.  Signatures as the HIP runtime's registration entry
 * points (pointer arguments of HIP types taken as void*).
 */
#include <stddef.h>

static void* g_handle = NULL;

void** __hipRegisterFatBinary(const void* data)
{
    (void)data;
    return &g_handle;
}

void __hipUnregisterFatBinary(void** modules) { (void)modules; }

void __hipRegisterFunction(void** modules, const void* host_fn, char* device_fn, const char* device_name,
                           unsigned int thread_limit, void* tid, void* bid, void* block_dim, void* grid_dim,
                           int* wsize)
{
    (void)modules; (void)host_fn; (void)device_fn; (void)device_name; (void)thread_limit;
    (void)tid; (void)bid; (void)block_dim; (void)grid_dim; (void)wsize;
}

void __hipRegisterVar(void** modules, void* var, char* host_var, char* device_var, int ext, size_t size,
                      int constant, int global)
{
    (void)modules; (void)var; (void)host_var; (void)device_var; (void)ext; (void)size; (void)constant;
    (void)global;
}
