/* Python entry point for vitattn_fwd with vectorcall argument passing.
 *
 * _vitattn_ext.vitattn_fwd(qkv_or_q, k, v, out, B, H, N, D, scale, layout,
 * stream) -> int status takes the same eleven arguments as the C function
 * declared in vitattn.h, in the same order: device addresses and the stream
 * handle as Python ints (or None for NULL), sizes and layout as ints, scale as
 * a float or an int.  It converts them and calls vitattn_fwd, nothing else:
 * every check and the launch happen in the library, and the status comes back
 * unchanged (0 = queued).  A wrong argument count or an argument of the wrong
 * Python type or range raises TypeError or OverflowError before the library
 * is called.
 *
 * ctypes spends about 2 us per call converting eleven arguments, which is
 * half the run time of a short attention call; this module spends a few
 * hundred nanoseconds, so a loop of prepared calls is bound by the GPU.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "vitattn.h"

/* None -> NULL, int -> its value as an address */
static int to_ptr(PyObject* o, void** p) {
  if (o == Py_None) {
    *p = NULL;
    return 0;
  }
  if (!PyLong_Check(o)) {
    PyErr_SetString(PyExc_TypeError, "device addresses and the stream must be int or None");
    return -1;
  }
  /* negative or wider than 64 bits: OverflowError */
  const unsigned long long x = PyLong_AsUnsignedLongLong(o);
  if (x == (unsigned long long)-1 && PyErr_Occurred()) return -1;
  *p = (void*)(uintptr_t)x;
  return 0;
}

static int to_int(PyObject* o, int* v) {
  if (!PyLong_Check(o)) {
    PyErr_SetString(PyExc_TypeError, "sizes and layout must be int");
    return -1;
  }
  const long x = PyLong_AsLong(o);
  if (x == -1 && PyErr_Occurred()) return -1;
  if (x < -2147483647L - 1 || x > 2147483647L) {
    PyErr_SetString(PyExc_OverflowError, "size or layout out of int range");
    return -1;
  }
  *v = (int)x;
  return 0;
}

static PyObject* py_vitattn_fwd(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  (void)self;
  if (nargs != 11) {
    PyErr_Format(PyExc_TypeError, "vitattn_fwd takes 11 arguments (%zd given)", nargs);
    return NULL;
  }
  void *q, *k, *v, *out, *stream;
  int sz[6];
  if (to_ptr(args[0], &q) || to_ptr(args[1], &k) || to_ptr(args[2], &v) || to_ptr(args[3], &out) ||
      to_ptr(args[10], &stream))
    return NULL;
  for (int i = 0; i < 4; ++i)
    if (to_int(args[4 + i], &sz[i])) return NULL;
  if (to_int(args[9], &sz[4])) return NULL;
  const double scale = PyFloat_AsDouble(args[8]);
  if (scale == -1.0 && PyErr_Occurred()) return NULL;
  const int status = vitattn_fwd(q, k, v, out, sz[0], sz[1], sz[2], sz[3], (float)scale, sz[4], stream);
  return PyLong_FromLong(status);
}

static PyMethodDef methods[] = {
    {"vitattn_fwd", (PyCFunction)(void (*)(void))py_vitattn_fwd, METH_FASTCALL,
     "vitattn_fwd(qkv_or_q, k, v, out, B, H, N, D, scale, layout, stream) -> status"},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_vitattn_ext",
                                    "vitattn_fwd of libvitattn.so with vectorcall arguments", -1, methods};

PyMODINIT_FUNC PyInit__vitattn_ext(void) { return PyModule_Create(&module); }
