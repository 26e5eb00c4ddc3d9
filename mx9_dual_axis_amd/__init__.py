"""placeholder; replaced by the binding"""
