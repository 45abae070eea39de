"""Placeholder; replaced by the ctypes binding of libmmf.so."""


def load():
    raise RuntimeError("libmmf.so binding not built yet")
